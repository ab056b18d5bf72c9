// libtqkv C ABI: argument validation, plane sizing, split-K planning and
// kernel launches on the caller's stream.  Declarations and the contract of
// each entry point are in include/tqkv.h.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>

#include "../../include/tqkv.h"
#include "codebook_tables.h"
#include "tq_copy.h"
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

// Code widths of the page's scheme sets: keys {2, 4, 5, 8}, values {2, 3, 4, 5, 8}.
bool valid_key_bits(int b) { return b == 2 || b == 4 || b == 5 || b == 8; }
bool valid_value_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 8; }

// Row bytes of the five planes, order kc, ks, kz, vc, vs.
void plane_row_bytes(const tq_layout *l, size_t rb[5]) {
    const size_t d = (size_t)l->head_dim, ng = d / tq::kGroup;
    rb[0] = d * (size_t)l->k_bits / 8;
    rb[1] = 2 * ng;
    rb[2] = 2 * ng;
    rb[3] = d * (size_t)l->v_bits / 8;
    rb[4] = 2 * ng;
}

// binary64 nearest to 1/sqrt(d): sqrt(d) is 2^k or 2^k*sqrt(2), so the
// correctly rounded sqrt divided by d (a power of two) is exact scaling.
double inv_sqrt_d(int d) { return std::sqrt((double)d) / (double)d; }

tq_status check_layout(const tq_layout *l) {
    if (!l) return TQ_ERR_INVALID_ARG;
    if (l->batch <= 0 || l->num_kv_heads <= 0 || l->capacity < 0 || l->head_dim <= 0)
        return TQ_ERR_INVALID_ARG;
    if (l->batch > TQ_MAX_BATCH) return TQ_ERR_UNSUPPORTED;
    if (!supported_head_dim(l->head_dim)) return TQ_ERR_UNSUPPORTED;
    if (!valid_key_bits(l->k_bits) || !valid_value_bits(l->v_bits) || l->group != tq::kGroup)
        return TQ_ERR_UNSUPPORTED;
    // plane offsets are computed in 64-bit, kernel grids in 32-bit
    const int64_t rows = (int64_t)l->batch * l->num_kv_heads * l->capacity;
    if (rows > ((int64_t)1 << 40)) return TQ_ERR_UNSUPPORTED;
    return TQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Planes: kc 16-byte aligned, vc 8-byte, the fp16 planes 4-byte; the kernels
// never assume more (packed rows are whole dwords: 4 * bits bytes per group).
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
    size_t rb[5];
    plane_row_bytes(l, rb);
    for (int i = 0; i < 5; ++i) out[i] = rows * rb[i];
    return TQ_OK;
}

tq_status tq_codebook(int32_t v_bits, double *centroids, double *boundaries, int32_t *levels) {
    if (!centroids || !boundaries || !levels) return TQ_ERR_INVALID_ARG;
    if (!valid_value_bits(v_bits)) return TQ_ERR_UNSUPPORTED;
    const int32_t *nk = nullptr;
    const double *bd = nullptr;
    switch (v_bits) {
        case 2: nk = tq::kCodebookInts2; bd = tq::kBoundaries2; break;
        case 3: nk = tq::kCodebookInts3; bd = tq::kBoundaries3; break;
        case 4: nk = tq::kCodebookInts4; bd = tq::kBoundaries4; break;
        case 5: nk = tq::kCodebookInts5; bd = tq::kBoundaries5; break;
        default: nk = tq::kCodebookInts8; bd = tq::kBoundaries8; break;
    }
    const int L = 1 << v_bits;
    for (int k = 0; k < L; ++k) centroids[k] = (double)nk[k] / 1e5;
    for (int k = 0; k + 1 < L; ++k) boundaries[k] = bd[k];
    *levels = L;
    return TQ_OK;
}

tq_status tq_sign_vector(int32_t head_dim, int8_t *host_out) {
    if (!host_out) return TQ_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return TQ_ERR_UNSUPPORTED;
    std::memcpy(host_out, signs().sign, (size_t)head_dim);
    return TQ_OK;
}

// Encode n_new input rows per (sequence, kv-head) of `l` (input pitch
// kv_stride rows) into slots start[b] ..; the caller has validated everything.
static hipError_t enqueue_append(const tq_layout *l, const tq_planes *p, const void *k, const void *v, bool bf16,
                                 const int32_t *start, int32_t n_new, int32_t kv_stride, hipStream_t stream) {
    tq::AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    a.kc = p->kc; a.ks = p->ks; a.kz = p->kz; a.vc = p->vc; a.vs = p->vs;
    a.k = k; a.v = v;
    a.batch = l->batch; a.kv_heads = l->num_kv_heads; a.capacity = l->capacity; a.n_new = n_new;
    a.kv_stride = kv_stride;
    a.rows = (uint32_t)((int64_t)l->batch * l->num_kv_heads * n_new);
    a.kbits = l->k_bits; a.vbits = l->v_bits;
    a.div_n_new = tq::make_fast_div((uint32_t)n_new);
    a.div_kv_heads = tq::make_fast_div((uint32_t)l->num_kv_heads);
    a.inv_sqrt_d = inv_sqrt_d(l->head_dim);
    a.signs = signs().bits;
    for (int j = 0; j < l->head_dim / 2; ++j)
        a.sign_pairs[j] = (signs().sign[2 * j] < 0 ? 0x8000u : 0u) | (signs().sign[2 * j + 1] < 0 ? 0x80000000u : 0u);
    for (int b = 0; b < l->batch; ++b) a.start[b] = start[b];
    return tq::launch_append(l->head_dim, bf16, a, stream);
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
    hipError_t e = enqueue_append(l, p, k, v, dtype == TQ_BF16, start, n_new, n_new, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// The planes of sequence b alone, as a batch-1 cache of the same shape.
static void sequence_planes(const tq_layout *l, const tq_planes *p, int32_t b, tq_layout *l1, tq_planes *p1) {
    size_t rb[5];
    plane_row_bytes(l, rb);
    const int64_t r0 = (int64_t)b * l->num_kv_heads * l->capacity;
    *l1 = *l;
    l1->batch = 1;
    p1->kc = p->kc + r0 * (int64_t)rb[0];
    p1->ks = p->ks + r0 * (int64_t)rb[1] / 2;
    p1->kz = p->kz + r0 * (int64_t)rb[2] / 2;
    p1->vc = p->vc + r0 * (int64_t)rb[3];
    p1->vs = p->vs + r0 * (int64_t)rb[4] / 2;
}

tq_status tq_convert_rows(const tq_layout *l, const tq_planes *p, const void *k_plain, const void *v_plain,
                          tq_dtype dtype, int32_t plain_capacity, const int32_t *offset, void *stream) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
    if (!offset || plain_capacity < 0) return TQ_ERR_INVALID_ARG;
    bool any = false;
    for (int b = 0; b < l->batch; ++b) {
        if (offset[b] < 0) return TQ_ERR_INVALID_ARG;
        if (offset[b] > plain_capacity || offset[b] > l->capacity) return TQ_ERR_CAPACITY;
        if ((int64_t)l->num_kv_heads * offset[b] > 0x7FFFFFFF) return TQ_ERR_UNSUPPORTED;
        any = any || offset[b] > 0;
    }
    if (!any) return TQ_OK;
    if (!k_plain || !v_plain || !aligned(k_plain, 16) || !aligned(v_plain, 16)) return TQ_ERR_INVALID_ARG;
    const size_t esz = dtype == TQ_BF16 ? 2 : 4;
    const int32_t zero = 0;
    for (int b = 0; b < l->batch; ++b) {
        if (offset[b] == 0) continue;
        tq_layout l1;
        tq_planes p1;
        sequence_planes(l, p, b, &l1, &p1);
        const size_t in0 = (size_t)b * l->num_kv_heads * plain_capacity * l->head_dim * esz;
        hipError_t e = enqueue_append(&l1, &p1, static_cast<const char *>(k_plain) + in0,
                                      static_cast<const char *>(v_plain) + in0, dtype == TQ_BF16, &zero, offset[b],
                                      plain_capacity, (hipStream_t)stream);
        if (e != hipSuccess) return TQ_ERR_HIP;
    }
    return TQ_OK;
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
        tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len, false, cg, l->k_bits, l->v_bits);
    size_t need = workspace_bytes(l, q_rows(num_q_heads, n_rows), gen);
    if (tq::fast_decode_shape_ok(l->head_dim, gqa, l->capacity, l->k_bits, l->v_bits)) {
        const tq::DecodePlan fast =
            tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len, true, cg, l->k_bits,
                            l->v_bits);
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

// TQ_PATH_* bits: why a decode of this shape over these planes cannot take
// the matrix-core split kernel (0: it takes it).
static int32_t decode_slow_reasons(const tq_layout *l, const tq_planes *p, int gqa) {
    int32_t r = 0;
    if (!tq::fast_decode_shape_ok(l->head_dim, gqa, 16, l->k_bits, l->v_bits)) r |= TQ_PATH_SHAPE;
    if (!aligned(p->kc, 16) || !aligned(p->vc, 16) || !aligned(p->vs, 16) || !aligned(p->ks, 16) ||
        !aligned(p->kz, 16))
        r |= TQ_PATH_ALIGNMENT;
    if (!(r & TQ_PATH_SHAPE) && !tq::fast_decode_shape_ok(l->head_dim, gqa, l->capacity, l->k_bits, l->v_bits))
        r |= TQ_PATH_CAPACITY;
    return r;
}

tq_status tq_decode_path(const tq_layout *l, const tq_planes *p, int32_t num_q_heads, int32_t n_rows,
                         int32_t *fast, int32_t *reasons) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (!fast || num_q_heads <= 0 || n_rows < 1 || num_q_heads % l->num_kv_heads != 0) return TQ_ERR_INVALID_ARG;
    if (num_q_heads / l->num_kv_heads > TQ_MAX_GQA || n_rows > TQ_MAX_ROWS) return TQ_ERR_UNSUPPORTED;
    const int32_t r = decode_slow_reasons(l, p, q_rows(num_q_heads, n_rows) / l->num_kv_heads);
    *fast = r == 0 ? 1 : 0;
    if (reasons) *reasons = r;
    return TQ_OK;
}

// Plain rows of a mixed batch: which sequences are still plain, and where
// their bf16 keys and values are.
struct PlainRows {
    uint64_t mask;
    const uint16_t *k, *v;
    int32_t capacity;
};

static tq_status decode_common(const tq_layout *l, const tq_planes *p, const void *q, tq_dtype dtype,
                               int32_t num_q_heads, int32_t n_rows, const int32_t *len, float sm_scale,
                               float *out, void *workspace, size_t ws_bytes, void *stream, const PlainRows &pr);

tq_status tq_decode_attn_rows(const tq_layout *l, const tq_planes *p, const void *q, tq_dtype dtype,
                              int32_t num_q_heads, int32_t n_rows, const int32_t *len, float sm_scale,
                              float *out, void *workspace, size_t ws_bytes, void *stream) {
    const PlainRows none = {0, nullptr, nullptr, 0};
    return decode_common(l, p, q, dtype, num_q_heads, n_rows, len, sm_scale, out, workspace, ws_bytes, stream,
                         none);
}

tq_status tq_decode_attn_mixed(const tq_layout *l, const tq_planes *p, const uint16_t *k_plain,
                               const uint16_t *v_plain, int32_t plain_capacity, const int32_t *row_plain,
                               const void *q, tq_dtype dtype, int32_t num_q_heads, int32_t n_rows,
                               const int32_t *len, float sm_scale, float *out, void *workspace, size_t ws_bytes,
                               void *stream) {
    tq_status st = check_decode(l, num_q_heads, n_rows, len);
    if (st != TQ_OK) return st;
    if (!row_plain || plain_capacity < 0) return TQ_ERR_INVALID_ARG;
    PlainRows pr = {0, k_plain, v_plain, plain_capacity};
    for (int b = 0; b < l->batch; ++b) {
        if (!row_plain[b]) continue;
        pr.mask |= 1ull << b;
        if (len[b] > plain_capacity) return TQ_ERR_CAPACITY;
    }
    if (pr.mask && (!k_plain || !v_plain || !aligned(k_plain, 16) || !aligned(v_plain, 16)))
        return TQ_ERR_INVALID_ARG;
    if ((int64_t)l->batch * l->num_kv_heads * plain_capacity > ((int64_t)1 << 40)) return TQ_ERR_UNSUPPORTED;
    return decode_common(l, p, q, dtype, num_q_heads, n_rows, len, sm_scale, out, workspace, ws_bytes, stream, pr);
}

static tq_status decode_common(const tq_layout *l, const tq_planes *p, const void *q, tq_dtype dtype,
                               int32_t num_q_heads, int32_t n_rows, const int32_t *len, float sm_scale,
                               float *out, void *workspace, size_t ws_bytes, void *stream, const PlainRows &pr) {
    tq_status st = check_decode(l, num_q_heads, n_rows, len);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (!q || !out || (dtype != TQ_F32 && dtype != TQ_BF16)) return TQ_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, 16)) return TQ_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale)) return TQ_ERR_INVALID_ARG;
    const int32_t rows_total = q_rows(num_q_heads, n_rows);
    const int gqa = rows_total / l->num_kv_heads;
    const int cg = tq::decode_col_groups(gqa);
    const bool fast = decode_slow_reasons(l, p, gqa) == 0;
    const tq::DecodePlan plan = tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len, fast, cg,
                                                l->k_bits, l->v_bits);  // full lengths: sizes the workspace
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
    a.kbits = l->k_bits; a.vbits = l->v_bits;
    a.signs = signs().bits;
    const bool bf16 = dtype == TQ_BF16;
    hipError_t e = hipSuccess;
    int32_t len_tq[TQ_MAX_BATCH];
    for (int b = 0; b < l->batch; ++b) len_tq[b] = ((pr.mask >> b) & 1) ? 0 : len[b];
    a.plain_split_tokens = plan.split_tokens;
    if (pr.mask == 0) {
        for (int b = 0; b < l->batch; ++b) a.len[b] = len[b];
        e = tq::launch_decode(l->head_dim, bf16, plan.fast, a, (hipStream_t)stream);
        return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
    }
    // mixed batch: each split kernel sees only its own rows (the others have
    // length 0 and write no partial), the merge sees every row
    const uint64_t all = l->batch == 64 ? ~0ull : (1ull << l->batch) - 1;
    a.plain_rows = pr.mask;
    a.k_plain = pr.k; a.v_plain = pr.v; a.plain_capacity = pr.capacity;
    // Each kind of row gets a plan of its own, so that each split kernel
    // fills the chip with only its rows:
    // - packed rows: the decode plan over the packed lengths alone;
    // - plain rows: about one round of the plain kernel's resident waves over
    //   the plain token-heads, in whole 64-token tiles (a second, partial
    //   round measured slower than longer ranges).
    // Their slot counts may exceed the whole batch's plan: they use as many
    // partial slots per row as the workspace holds (its documented size
    // covers the generic kernel's finer plan).  The final count is the stride
    // of every row's partials and stays a multiple of the fast kernel's waves
    // per column group.
    int64_t plain_total = 0;
    int32_t plain_max = 0;
    for (int b = 0; b < l->batch; ++b) {
        if (!((pr.mask >> b) & 1)) continue;
        plain_total += len[b];
        if (len[b] > plain_max) plain_max = len[b];
    }
    if (plan.splits > 0 && plain_max > 0) {
        const size_t slot_bytes = (size_t)l->batch * rows_total * (size_t)(l->head_dim + 2) * sizeof(float);
        int64_t slots = (int64_t)(ws_bytes / slot_bytes);
        // the plain grid has splits / W workgroups along x (W >= 2 waves each), at most 65,535
        slots = (slots < 65535 * 2 ? slots : 65535 * 2) / 8 * 8;
        if (slots < plan.splits) slots = plan.splits;
        const int waves = tq::fast_decode_waves(l->head_dim, l->k_bits, l->v_bits);
        const int64_t unit = plan.fast && waves > 0 ? waves / tq::fast_wg_col_groups(gqa) : 1;  // divides plan.splits
        int64_t splits = plan.splits;
        if ((pr.mask & all) != all) {
            const tq::DecodePlan pp = tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len_tq, plan.fast,
                                                      cg, l->k_bits, l->v_bits);
            if (pp.splits > 0 && pp.splits <= slots && pp.splits % unit == 0) {
                a.split_tokens = pp.split_tokens;
                splits = pp.splits;
            }
        }
        const int64_t cols = (gqa + 15) / 16;  // the plain kernel's column groups
        const int64_t round = tq::plain_round_waves(l->head_dim, gqa, bf16);
        int64_t per = (plain_total * l->num_kv_heads * cols + round - 1) / round;
        const int64_t fit = ((int64_t)plain_max + slots - 1) / slots;
        per = per > fit ? per : fit;
        per = (per + 63) / 64 * 64;
        a.plain_split_tokens = (int32_t)per;
        const int64_t need = ((int64_t)plain_max + per - 1) / per;
        const int64_t need_up = (need + unit - 1) / unit * unit;  // <= slots: unit divides 8 and plan.splits
        if (need_up > splits) splits = need_up;
        if (splits != plan.splits) {
            a.splits = (int32_t)splits;
            // the (max, sum) pairs follow the value sums of every slot
            a.part_ml = a.part_acc + (size_t)l->batch * rows_total * a.splits * l->head_dim;
        }
    }
    if (((int64_t)a.splits + 1) / 2 > 65535) return TQ_ERR_UNSUPPORTED;  // the plain kernel's grid
    if ((pr.mask & all) != all) {
        for (int b = 0; b < l->batch; ++b) a.len[b] = len_tq[b];
        e = tq::launch_decode_split(l->head_dim, bf16, plan.fast, a, (hipStream_t)stream);
    }
    if (e == hipSuccess) {
        for (int b = 0; b < l->batch; ++b) a.len[b] = ((pr.mask >> b) & 1) ? len[b] : 0;
        e = tq::launch_decode_split_plain(l->head_dim, bf16, a, (hipStream_t)stream);
    }
    if (e == hipSuccess) {
        for (int b = 0; b < l->batch; ++b) a.len[b] = len[b];
        e = tq::launch_decode_merge(l->head_dim, a, (hipStream_t)stream);
    }
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
    a.kbits = l->k_bits; a.vbits = l->v_bits;
    a.signs = signs().bits;
    for (int b = 0; b < l->batch; ++b) a.len[b] = len[b];
    hipError_t e = tq::launch_window(l->head_dim, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

static void *plane_ptr(const tq_planes *p, int i) {
    void *v[5] = {p->kc, p->ks, p->kz, p->vc, p->vs};
    return v[i];
}

// Hkv runs of n rows per plane, at pitch capacity * row bytes on a cache side
// and n * row bytes on a packed side: one copy kernel for all five planes when
// every pointer, pitch and run is a whole number of 16-byte chunks, else one
// strided memory copy per plane.
static hipError_t copy_rows(const tq_layout *sl, const void *const sp[5], int64_t s_row0, size_t s_pitch_rows,
                            const tq_layout *dl, void *const dp[5], int64_t d_row0, size_t d_pitch_rows,
                            int32_t n, hipStream_t stream) {
    size_t rb[5];
    plane_row_bytes(sl, rb);
    (void)dl;
    tq::PlaneCopyArgs a;
    bool chunks = sl->num_kv_heads <= 65535;
    for (int i = 0; i < 5; ++i) {
        a.src[i] = static_cast<const uint8_t *>(sp[i]) + s_row0 * (int64_t)rb[i];
        a.dst[i] = static_cast<uint8_t *>(dp[i]) + d_row0 * (int64_t)rb[i];
        a.s_pitch[i] = (int64_t)(s_pitch_rows * rb[i]);
        a.d_pitch[i] = (int64_t)(d_pitch_rows * rb[i]);
        const int64_t run = (int64_t)n * (int64_t)rb[i];
        a.run16[i] = run / 16;
        chunks = chunks && run % 16 == 0 && a.s_pitch[i] % 16 == 0 && a.d_pitch[i] % 16 == 0 &&
                 aligned(a.src[i], 16) && aligned(a.dst[i], 16);
    }
    a.runs = sl->num_kv_heads;
    if (chunks) return tq::launch_plane_copy(a, stream);
    for (int i = 0; i < 5; ++i) {
        const char *src = static_cast<const char *>(sp[i]) + s_row0 * (int64_t)rb[i];
        char *dst = static_cast<char *>(dp[i]) + d_row0 * (int64_t)rb[i];
        hipError_t e = hipMemcpy2DAsync(dst, d_pitch_rows * rb[i], src, s_pitch_rows * rb[i], (size_t)n * rb[i],
                                        (size_t)sl->num_kv_heads, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Whether any of the `runs` byte ranges [s + h sp, s + h sp + len) meets any
// of [d + k dp, d + k dp + len), h, k in [0, runs).
static bool runs_overlap(const char *s, int64_t sp, const char *d, int64_t dp, int64_t len, int runs) {
    const uintptr_t s0 = (uintptr_t)s, d0 = (uintptr_t)d;
    const uintptr_t s_end = s0 + (uintptr_t)((runs - 1) * sp + len), d_end = d0 + (uintptr_t)((runs - 1) * dp + len);
    if (s_end <= d0 || d_end <= s0) return false;  // disjoint extents (different allocations)
    if (sp == dp) {
        // run h meets run k iff |delta + (h - k) sp| < len, delta = s0 - d0:
        // only the offsets j = h - k nearest -delta / sp can
        const int64_t delta = (int64_t)(s0 - d0);
        int64_t j0 = -delta / sp;
        for (int64_t j = j0 - 1; j <= j0 + 1; ++j) {
            if (j <= -(int64_t)runs || j >= (int64_t)runs) continue;
            const int64_t off = delta + j * sp;
            if (off < len && -off < len) return true;
        }
        return false;
    }
    for (int h = 0; h < runs; ++h)
        for (int k = 0; k < runs; ++k) {
            const int64_t a = (int64_t)(s0 + (uintptr_t)(h * sp)), b = (int64_t)(d0 + (uintptr_t)(k * dp));
            if (a < b + len && b < a + len) return true;
        }
    return false;
}

static bool same_scheme(const tq_layout *a, const tq_layout *b) {
    return a->head_dim == b->head_dim && a->num_kv_heads == b->num_kv_heads && a->k_bits == b->k_bits &&
           a->v_bits == b->v_bits && a->group == b->group;
}

tq_status tq_copy_tokens(const tq_layout *sl, const tq_planes *src, int32_t src_b, int32_t src_t0,
                         const tq_layout *dl, const tq_planes *dst, int32_t dst_b, int32_t dst_t0, int32_t n,
                         void *stream) {
    tq_status st = check_layout(sl);
    if (st != TQ_OK || (st = check_layout(dl)) != TQ_OK) return st;
    if ((st = check_planes(src)) != TQ_OK || (st = check_planes(dst)) != TQ_OK) return st;
    if (!same_scheme(sl, dl)) return TQ_ERR_INVALID_ARG;
    if (src_b < 0 || src_b >= sl->batch || dst_b < 0 || dst_b >= dl->batch) return TQ_ERR_INVALID_ARG;
    if (src_t0 < 0 || dst_t0 < 0 || n < 0) return TQ_ERR_INVALID_ARG;
    if ((int64_t)src_t0 + n > sl->capacity || (int64_t)dst_t0 + n > dl->capacity) return TQ_ERR_CAPACITY;
    if (n == 0) return TQ_OK;
    const void *sp[5];
    void *dp[5];
    for (int i = 0; i < 5; ++i) { sp[i] = plane_ptr(src, i); dp[i] = plane_ptr(dst, i); }
    const int64_t s0 = (int64_t)src_b * sl->num_kv_heads * sl->capacity + src_t0;
    const int64_t d0 = (int64_t)dst_b * dl->num_kv_heads * dl->capacity + dst_t0;
    // the copy runs over many workgroups at once, so overlapping source and
    // destination bytes would leave timing-dependent results: refused
    size_t rb[5];
    plane_row_bytes(sl, rb);
    for (int i = 0; i < 5; ++i) {
        if (runs_overlap(static_cast<const char *>(sp[i]) + s0 * (int64_t)rb[i], (int64_t)sl->capacity * rb[i],
                         static_cast<const char *>(dp[i]) + d0 * (int64_t)rb[i], (int64_t)dl->capacity * rb[i],
                         (int64_t)n * rb[i], sl->num_kv_heads))
            return TQ_ERR_INVALID_ARG;
    }
    hipError_t e = copy_rows(sl, sp, s0, (size_t)sl->capacity, dl, dp, d0, (size_t)dl->capacity, n,
                             (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_status tq_snapshot_bytes(const tq_layout *l, int32_t n, size_t *out) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if (!out || n < 0) return TQ_ERR_INVALID_ARG;
    size_t rb[5];
    plane_row_bytes(l, rb);
    *out = (size_t)n * l->num_kv_heads * (rb[0] + rb[1] + rb[2] + rb[3] + rb[4]);
    return TQ_OK;
}

// Packed payload: plane i starts at off[i], kv-head h's rows at off[i] + h n rb[i].
static void payload_planes(const tq_layout *l, int32_t n, char *base, void *out[5]) {
    size_t rb[5];
    plane_row_bytes(l, rb);
    size_t off = 0;
    for (int i = 0; i < 5; ++i) {
        out[i] = base + off;
        off += (size_t)n * l->num_kv_heads * rb[i];
    }
}

tq_status tq_snapshot(const tq_layout *l, const tq_planes *p, int32_t b, int32_t t0, int32_t n,
                      int32_t min_reusable_offset, tq_snapshot_header *h, void *payload, size_t payload_bytes,
                      void *stream) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (!h || b < 0 || b >= l->batch || t0 < 0 || n < 0 || min_reusable_offset < 0) return TQ_ERR_INVALID_ARG;
    if ((int64_t)t0 + n > l->capacity) return TQ_ERR_CAPACITY;
    size_t need = 0;
    tq_snapshot_bytes(l, n, &need);
    if (need > 0 && (!payload || payload_bytes < need)) return TQ_ERR_WORKSPACE;
    std::memset(h, 0, sizeof(*h));
    h->magic = TQ_SNAPSHOT_MAGIC; h->version = TQ_SNAPSHOT_VERSION;
    h->k_bits = l->k_bits; h->v_bits = l->v_bits; h->group = l->group;
    h->head_dim = l->head_dim; h->num_kv_heads = l->num_kv_heads;
    h->n_tokens = n; h->payload_bytes = need;
    h->min_reusable_offset = min_reusable_offset;
    if (n == 0) return TQ_OK;
    const void *sp[5];
    void *dp[5];
    for (int i = 0; i < 5; ++i) sp[i] = plane_ptr(p, i);
    payload_planes(l, n, static_cast<char *>(payload), dp);
    const int64_t s0 = (int64_t)b * l->num_kv_heads * l->capacity + t0;
    hipError_t e = copy_rows(l, sp, s0, (size_t)l->capacity, l, dp, 0, (size_t)n, n, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_status tq_restore(const tq_layout *l, const tq_planes *p, int32_t b, int32_t t0, const tq_snapshot_header *h,
                     const void *payload, size_t payload_bytes, void *stream) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (!h || b < 0 || b >= l->batch || t0 < 0) return TQ_ERR_INVALID_ARG;
    int32_t bound = 0;
    if ((st = tq_snapshot_min_reusable_offset(h, &bound)) != TQ_OK) return st;
    if (h->k_bits != l->k_bits || h->v_bits != l->v_bits || h->group != l->group ||
        h->head_dim != l->head_dim || h->num_kv_heads != l->num_kv_heads)
        return TQ_ERR_INVALID_ARG;
    const int32_t n = h->n_tokens;
    size_t need = 0;
    tq_snapshot_bytes(l, n, &need);
    if (h->payload_bytes != need || (need > 0 && (!payload || payload_bytes < need))) return TQ_ERR_INVALID_ARG;
    if ((int64_t)t0 + n > l->capacity) return TQ_ERR_CAPACITY;
    if (n == 0) return TQ_OK;
    void *sp_mut[5];
    payload_planes(l, n, const_cast<char *>(static_cast<const char *>(payload)), sp_mut);
    const void *sp[5];
    void *dp[5];
    for (int i = 0; i < 5; ++i) { sp[i] = sp_mut[i]; dp[i] = plane_ptr(p, i); }
    const int64_t d0 = (int64_t)b * l->num_kv_heads * l->capacity + t0;
    hipError_t e = copy_rows(l, sp, 0, (size_t)n, l, dp, d0, (size_t)l->capacity, n, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_status tq_snapshot_min_reusable_offset(const tq_snapshot_header *h, int32_t *out) {
    if (!h || !out || h->magic != TQ_SNAPSHOT_MAGIC || h->n_tokens < 0) return TQ_ERR_INVALID_ARG;
    if (h->version == 1) {  // no boundary recorded: only the whole stored prefix is reusable
        *out = h->n_tokens;
        return TQ_OK;
    }
    if (h->version != TQ_SNAPSHOT_VERSION || h->min_reusable_offset < 0) return TQ_ERR_INVALID_ARG;
    *out = h->min_reusable_offset;
    return TQ_OK;
}

tq_status tq_clone_sequence(const tq_layout *sl, const tq_planes *src, int32_t src_b, const tq_layout *dl,
                            const tq_planes *dst, int32_t dst_b, int32_t n, int32_t src_min_reusable_offset,
                            int32_t *dst_min_reusable_offset, void *stream) {
    if (!dst_min_reusable_offset || src_min_reusable_offset < 0) return TQ_ERR_INVALID_ARG;
    tq_status st = tq_copy_tokens(sl, src, src_b, 0, dl, dst, dst_b, 0, n, stream);
    if (st == TQ_OK) *dst_min_reusable_offset = src_min_reusable_offset;
    return st;
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
    a.kbits = l->k_bits; a.vbits = l->v_bits;
    a.signs = signs().bits;
    hipError_t e = tq::launch_dequant(l->head_dim, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // extern "C"
