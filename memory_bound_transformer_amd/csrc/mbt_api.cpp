// mbt_api.cpp -- the extern "C" boundary of libmbt (declared in include/mbt.h).
//
// Every entry point validates all of its arguments before touching a pointer
// or the HIP runtime ("thox-edge-ops v2", section 5.5: validate before any
// pointer arithmetic); a rejected call enqueues nothing and returns a status
// with a detail string in a thread-local buffer.  There is no fallback path.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "mbt.h"
#include "mbt_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

mbt_status fail(mbt_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

mbt_status ok() {
    g_last_error[0] = '\0';
    return MBT_OK;
}

int elt_bytes(int32_t dtype) { return dtype == MBT_F32 ? 4 : 2; }

bool valid_dtype(int32_t dtype) {
    return dtype == MBT_F32 || dtype == MBT_F16 || dtype == MBT_BF16;
}

bool finite_nonneg(float v) { return std::isfinite(v) && v >= 0.0f; }
bool finite_pos(float v) { return std::isfinite(v) && v > 0.0f; }

bool aligned(const void* p, int a) {
    return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0;
}

// Byte range of a tensor, for overlap checks.
struct Range {
    const char* p;
    int64_t n;
    const char* name;
};

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.n <= 0 || b.n <= 0) return false;
    return a.p < b.p + b.n && b.p < a.p + a.n;
}

// Inputs vs outputs: an output may coincide exactly with the one input it
// replaces (`same_ok`); any other overlap is an alias error.
mbt_status check_alias(const Range& out, const Range& in, bool same_ok) {
    if (!overlap(out, in)) return MBT_OK;
    if (same_ok && out.p == in.p && out.n == in.n) return MBT_OK;
    return fail(MBT_ERR_ALIAS, "%s overlaps %s", out.name, in.name);
}

// Heads per token (query or key) accepted by the prologue entry points: far
// above any model's, and small enough that every sum of head counts and
// every head index stays inside int32.
constexpr int32_t kMaxHeads = 1 << 20;

// Widest norm row (H) and activation half (d): every element and chunk index
// inside a row, rounded up to whole blocks, stays inside int32.
constexpr int32_t kMaxRow = 1 << 28;

// Safe product of non-negative sizes, or -1 past 2^62.
int64_t mul(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a != 0 && b > (INT64_C(1) << 62) / a) return -1;
    return a * b;
}

mbt_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MBT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A strided view: `rows` rows of `len` bytes, `stride` bytes apart.
struct View {
    const char* p;
    int64_t stride, len, rows;
    const char* name;
};

int64_t span(const View& v) { return v.rows > 0 ? (v.rows - 1) * v.stride + v.len : 0; }

int64_t floor_div(int64_t a, int64_t b) {     // b > 0
    const int64_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

// Do the two views share a byte?  Exact when the strides are equal (rows
// a + t s + [0, la) and b + u s + [0, lb) meet iff -lb < d + k s < la for
// some k = u - t in [-(ra - 1), rb - 1], d = b - a); otherwise the spans are
// compared, which may report an overlap of interleaved views.
bool views_overlap(const View& a, const View& b) {
    if (!a.p || !b.p || a.rows <= 0 || b.rows <= 0 || a.len <= 0 || b.len <= 0) return false;
    const intptr_t pa = reinterpret_cast<intptr_t>(a.p), pb = reinterpret_cast<intptr_t>(b.p);
    if (!(pa < pb + span(b) && pb < pa + span(a))) return false;
    if (a.stride != b.stride) return true;
    const int64_t s = a.stride, d = (int64_t)(pb - pa);
    int64_t k = floor_div(-b.len - d, s) + 1;          // least k with d + k s > -lb
    if (k < -(a.rows - 1)) k = -(a.rows - 1);
    return k <= b.rows - 1 && d + k * s < a.len;
}

bool same_view(const View& a, const View& b) {
    return a.p == b.p && a.len == b.len && a.rows == b.rows && (a.rows <= 1 || a.stride == b.stride);
}

// Everything the three QK-norm + RoPE entry points take; strides in elements.
struct QkCall {
    const void* q_in;
    const void* k_in;
    void* q_out;
    void* k_out;
    const void* w_q;
    const void* w_k;
    const float* cos_sin;
    int64_t max_pos;
    const int64_t* pos;
    int32_t Q, K;
    int64_t T;
    int32_t D, rot;
    float eps;
    int32_t weight_offset, layout, dtype, flags;
    int64_t q_in_st, k_in_st, q_out_st, k_out_st;
    const int64_t* slot;
    int64_t n_slots;
    const void* v_in;
    void* v_out;
    int64_t v_in_st, v_out_st;
};

// Validates a call completely, then launches.  Stride 0 means dense.
mbt_status qk_run(QkCall c, void* stream) {
    if (!valid_dtype(c.dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", c.dtype);
    if (c.layout != MBT_ROPE_ROTATE_HALF && c.layout != MBT_ROPE_INTERLEAVED)
        return fail(MBT_ERR_BAD_ENUM, "layout %d", c.layout);
    if (c.weight_offset != 0 && c.weight_offset != 1)
        return fail(MBT_ERR_BAD_ENUM, "weight_offset %d", c.weight_offset);
    if (c.flags & ~MBT_QK_ROUND_ONCE) return fail(MBT_ERR_BAD_ENUM, "flags 0x%x", c.flags);
    if (c.Q < 0 || c.K < 0 || c.Q > kMaxHeads || c.K > kMaxHeads || c.Q + c.K < 1)
        return fail(MBT_ERR_BAD_SHAPE, "Q=%d K=%d", c.Q, c.K);
    if (c.T < 0) return fail(MBT_ERR_BAD_SHAPE, "T=%lld", (long long)c.T);
    if (c.D < 1 || c.D > 512) return fail(MBT_ERR_BAD_SHAPE, "head_dim %d not in [1, 512]", c.D);
    if (c.rot < 0 || c.rot > c.D || (c.rot % 2) != 0)
        return fail(MBT_ERR_BAD_SHAPE, "rot_dim %d (head_dim %d)", c.rot, c.D);
    if (!finite_nonneg(c.eps)) return fail(MBT_ERR_BAD_SCALAR, "eps must be finite and >= 0");
    if (c.max_pos < 0) return fail(MBT_ERR_BAD_SCALAR, "max_pos %lld", (long long)c.max_pos);
    if (c.n_slots < 0) return fail(MBT_ERR_BAD_SCALAR, "n_slots %lld", (long long)c.n_slots);
    const bool has_v = c.v_in != nullptr || c.v_out != nullptr;
    const int64_t qrow = (int64_t)c.Q * c.D, krow = (int64_t)c.K * c.D;
    int64_t* sts[] = {&c.q_in_st, &c.k_in_st, &c.q_out_st, &c.k_out_st, &c.v_in_st, &c.v_out_st};
    const int64_t need[] = {qrow, krow, qrow, krow, krow, krow};
    for (int i = 0; i < 6; ++i) {
        if (*sts[i] == 0) *sts[i] = need[i];
        if (*sts[i] < need[i] || *sts[i] > (INT64_C(1) << 40))
            return fail(MBT_ERR_BAD_SHAPE, "token stride %lld outside [%lld, 2^40]",
                        (long long)*sts[i], (long long)need[i]);
    }
    const int eb = elt_bytes(c.dtype);
    const int64_t out_rows = c.slot ? c.n_slots : c.T;
    auto view = [&](const void* p, int64_t st, int64_t len, int64_t rows, const char* n) {
        return View{(const char*)p, mul(st, eb), mul(len, eb), rows, n};
    };
    const View qi = view(c.Q ? c.q_in : nullptr, c.q_in_st, qrow, c.T, "q_in");
    const View ki = view(c.K ? c.k_in : nullptr, c.k_in_st, krow, c.T, "k_in");
    const View vi = view(has_v ? c.v_in : nullptr, c.v_in_st, krow, c.T, "v_in");
    const View qo = view(c.Q ? c.q_out : nullptr, c.q_out_st, qrow, c.T, "q_out");
    const View ko = view(c.K ? c.k_out : nullptr, c.k_out_st, krow, out_rows, "k_out");
    const View vo = view(has_v ? c.v_out : nullptr, c.v_out_st, krow, out_rows, "v_out");
    const int64_t cs_bytes = mul(mul(c.max_pos, c.rot), 4);
    for (const View* v : {&qi, &ki, &vi, &qo, &ko, &vo})
        if (v->stride < 0 || v->len < 0 || (v->rows > 0 && mul(v->rows, v->stride) < 0))
            return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    if (cs_bytes < 0 || mul(c.T, c.Q + c.K) > (INT64_C(1) << 40))
        return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    if (c.T == 0) return ok();
    const bool need_cache = c.rot > 0 && c.max_pos > 0;
    if (c.Q > 0 && (!c.q_in || !c.q_out || !c.w_q))
        return fail(MBT_ERR_NULL_POINTER, "q_in, q_out and w_q are required when Q > 0");
    if (c.K > 0 && (!c.k_in || !c.k_out || !c.w_k))
        return fail(MBT_ERR_NULL_POINTER, "k_in, k_out and w_k are required when K > 0");
    if (has_v && (!c.v_in || !c.v_out))
        return fail(MBT_ERR_NULL_POINTER, "v_in and v_out go together");
    if (!c.pos) return fail(MBT_ERR_NULL_POINTER, "pos is required");
    if (need_cache && !c.cos_sin)
        return fail(MBT_ERR_NULL_POINTER, "cos_sin is required when rot_dim > 0");
    if ((c.Q > 0 && (!aligned(c.q_in, eb) || !aligned(c.q_out, eb) || !aligned(c.w_q, eb))) ||
        (c.K > 0 && (!aligned(c.k_in, eb) || !aligned(c.k_out, eb) || !aligned(c.w_k, eb))) ||
        (has_v && (!aligned(c.v_in, eb) || !aligned(c.v_out, eb))) || !aligned(c.pos, 8) ||
        (c.slot && !aligned(c.slot, 8)) || (need_cache && !aligned(c.cos_sin, 4)))
        return fail(MBT_ERR_ALIGN, "a pointer is not aligned to its element size");
    const int64_t w_bytes = (int64_t)c.D * eb;
    const View wq{(const char*)(c.Q ? c.w_q : nullptr), w_bytes, w_bytes, 1, "w_q"};
    const View wk{(const char*)(c.K ? c.w_k : nullptr), w_bytes, w_bytes, 1, "w_k"};
    const View cs{(const char*)(need_cache ? c.cos_sin : nullptr), cs_bytes, cs_bytes, 1,
                  "cos_sin"};
    const View ps{(const char*)c.pos, c.T * 8, c.T * 8, 1, "pos"};
    const View sl{(const char*)c.slot, c.T * 8, c.T * 8, 1, "slot"};
    const View* ins[] = {&qi, &ki, &vi, &wq, &wk, &cs, &ps, &sl};
    const View* outs[] = {&qo, &ko, &vo};
    for (const View* o : outs) {
        for (const View* i : ins) {
            // the in-place form: an output exactly on the input it replaces
            // (not through a slot table, which could move rows onto others)
            const bool same_ok = !c.slot && ((o == &qo && i == &qi) || (o == &ko && i == &ki) ||
                                             (o == &vo && i == &vi));
            if (views_overlap(*o, *i) && !(same_ok && same_view(*o, *i)))
                return fail(MBT_ERR_ALIAS, "%s overlaps %s", o->name, i->name);
        }
    }
    if (views_overlap(qo, ko) || views_overlap(qo, vo) || views_overlap(ko, vo))
        return fail(MBT_ERR_ALIAS, "the outputs overlap each other");

    mbt::QkArgs a{};
    a.q_in = c.q_in; a.k_in = c.k_in; a.q_out = c.q_out; a.k_out = c.k_out;
    a.w_q = c.w_q; a.w_k = c.w_k; a.cos_sin = c.cos_sin; a.max_pos = c.max_pos; a.pos = c.pos;
    a.Q = c.Q; a.K = c.K; a.T = c.T; a.head_dim = c.D; a.rot_dim = c.rot; a.eps = c.eps;
    a.weight_offset = c.weight_offset; a.layout = c.layout; a.dtype = c.dtype;
    a.q_in_stride = c.q_in_st; a.k_in_stride = c.k_in_st;
    a.q_out_stride = c.q_out_st; a.k_out_stride = c.k_out_st;
    a.round_once = (c.flags & MBT_QK_ROUND_ONCE) != 0;
    a.slot = c.slot; a.n_slots = c.n_slots;
    a.v_in = has_v ? c.v_in : nullptr; a.v_out = has_v ? c.v_out : nullptr;
    a.v_in_stride = c.v_in_st; a.v_out_stride = c.v_out_st;
    return hip_status(mbt::launch_qknorm_rope(a, (hipStream_t)stream), "qknorm_rope launch");
}

}  // namespace

extern "C" {

int32_t mbt_abi_version(void) { return MBT_ABI_VERSION; }

const char* mbt_last_error(void) { return g_last_error; }

const char* mbt_status_string(mbt_status s) {
    switch (s) {
    case MBT_OK: return "MBT_OK";
    case MBT_ERR_NULL_POINTER: return "MBT_ERR_NULL_POINTER";
    case MBT_ERR_BAD_SHAPE: return "MBT_ERR_BAD_SHAPE";
    case MBT_ERR_BAD_DTYPE: return "MBT_ERR_BAD_DTYPE";
    case MBT_ERR_BAD_ENUM: return "MBT_ERR_BAD_ENUM";
    case MBT_ERR_BAD_SCALAR: return "MBT_ERR_BAD_SCALAR";
    case MBT_ERR_ALIAS: return "MBT_ERR_ALIAS";
    case MBT_ERR_HIP: return "MBT_ERR_HIP";
    case MBT_ERR_ALIGN: return "MBT_ERR_ALIGN";
    }
    return "MBT_ERR_UNKNOWN";
}

mbt_status mbt_qknorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                           const void* w_q, const void* w_k, const float* cos_sin,
                           int64_t max_pos, const int64_t* pos, int32_t Q, int32_t K,
                           int64_t T, int32_t head_dim, int32_t rot_dim, float eps,
                           int32_t weight_offset, int32_t layout, int32_t dtype,
                           void* stream) {
    QkCall c{};
    c.q_in = q_in; c.k_in = k_in; c.q_out = q_out; c.k_out = k_out; c.w_q = w_q; c.w_k = w_k;
    c.cos_sin = cos_sin; c.max_pos = max_pos; c.pos = pos; c.Q = Q; c.K = K; c.T = T;
    c.D = head_dim; c.rot = rot_dim; c.eps = eps; c.weight_offset = weight_offset;
    c.layout = layout; c.dtype = dtype;
    return qk_run(c, stream);
}

mbt_status mbt_qknorm_rope_ex(const void* q_in, const void* k_in, void* q_out, void* k_out,
                              const void* w_q, const void* w_k, const float* cos_sin,
                              int64_t max_pos, const int64_t* pos, int32_t Q, int32_t K,
                              int64_t T, int32_t head_dim, int32_t rot_dim, float eps,
                              int32_t weight_offset, int32_t layout, int32_t dtype,
                              int64_t q_in_stride, int64_t k_in_stride, int64_t q_out_stride,
                              int64_t k_out_stride, int32_t flags, void* stream) {
    QkCall c{};
    c.q_in = q_in; c.k_in = k_in; c.q_out = q_out; c.k_out = k_out; c.w_q = w_q; c.w_k = w_k;
    c.cos_sin = cos_sin; c.max_pos = max_pos; c.pos = pos; c.Q = Q; c.K = K; c.T = T;
    c.D = head_dim; c.rot = rot_dim; c.eps = eps; c.weight_offset = weight_offset;
    c.layout = layout; c.dtype = dtype; c.flags = flags;
    c.q_in_st = q_in_stride; c.k_in_st = k_in_stride;
    c.q_out_st = q_out_stride; c.k_out_st = k_out_stride;
    if (q_in_stride < 0 || k_in_stride < 0 || q_out_stride < 0 || k_out_stride < 0)
        return fail(MBT_ERR_BAD_SHAPE, "negative token stride");
    return qk_run(c, stream);
}

mbt_status mbt_qkv_norm_rope_cache(const void* qkv, void* q_out, void* k_cache, void* v_cache,
                                   const int64_t* slot, int64_t n_slots, const void* w_q,
                                   const void* w_k, const float* cos_sin, int64_t max_pos,
                                   const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                                   int32_t head_dim, int32_t rot_dim, float eps,
                                   int32_t weight_offset, int32_t layout, int32_t dtype,
                                   int32_t flags, void* stream) {
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (K < 1 || Q < 0 || Q > kMaxHeads || K > kMaxHeads)
        return fail(MBT_ERR_BAD_SHAPE, "Q=%d K=%d (a cache needs K >= 1)", Q, K);
    if (head_dim < 1 || head_dim > 512)
        return fail(MBT_ERR_BAD_SHAPE, "head_dim %d not in [1, 512]", head_dim);
    if (T > 0 && (!qkv || !k_cache || !v_cache || !slot))
        return fail(MBT_ERR_NULL_POINTER, "qkv, k_cache, v_cache and slot are required");
    const int eb = elt_bytes(dtype);
    const char* base = (const char*)qkv;
    const int64_t tok = ((int64_t)Q + 2 * (int64_t)K) * head_dim;   // elements per token
    QkCall c{};
    c.q_in = base; c.k_in = base ? base + (int64_t)Q * head_dim * eb : nullptr;
    c.v_in = base ? base + ((int64_t)Q + K) * head_dim * eb : nullptr;
    c.q_out = q_out; c.k_out = k_cache; c.v_out = v_cache;
    c.w_q = w_q; c.w_k = w_k; c.cos_sin = cos_sin; c.max_pos = max_pos; c.pos = pos;
    c.Q = Q; c.K = K; c.T = T; c.D = head_dim; c.rot = rot_dim; c.eps = eps;
    c.weight_offset = weight_offset; c.layout = layout; c.dtype = dtype; c.flags = flags;
    c.q_in_st = tok; c.k_in_st = tok; c.v_in_st = tok;
    c.slot = slot; c.n_slots = n_slots;
    if (T == 0) c.v_in = c.v_out = nullptr;
    return qk_run(c, stream);
}

mbt_status mbt_rope(void* q, void* k, const float* cos_sin, int64_t max_pos, const int64_t* pos,
                    int32_t Q, int32_t K, int64_t T, int32_t head_dim, int32_t rot_dim,
                    int32_t layout, int32_t dtype, void* stream) {
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (layout != MBT_ROPE_ROTATE_HALF && layout != MBT_ROPE_INTERLEAVED)
        return fail(MBT_ERR_BAD_ENUM, "layout %d", layout);
    if (Q < 0 || K < 0 || Q > kMaxHeads || K > kMaxHeads || Q + K < 1)
        return fail(MBT_ERR_BAD_SHAPE, "Q=%d K=%d", Q, K);
    if (T < 0) return fail(MBT_ERR_BAD_SHAPE, "T=%lld", (long long)T);
    if (head_dim < 1 || head_dim > 512)
        return fail(MBT_ERR_BAD_SHAPE, "head_dim %d not in [1, 512]", head_dim);
    if (rot_dim < 0 || rot_dim > head_dim || (rot_dim % 2) != 0)
        return fail(MBT_ERR_BAD_SHAPE, "rot_dim %d (head_dim %d)", rot_dim, head_dim);
    if (max_pos < 0) return fail(MBT_ERR_BAD_SCALAR, "max_pos %lld", (long long)max_pos);
    const int eb = elt_bytes(dtype);
    const int64_t q_bytes = mul(mul(mul(T, Q), head_dim), eb);
    const int64_t k_bytes = mul(mul(mul(T, K), head_dim), eb);
    const int64_t cs_bytes = mul(mul(max_pos, rot_dim), 4);
    if (q_bytes < 0 || k_bytes < 0 || cs_bytes < 0 || mul(T, Q + K) > (INT64_C(1) << 40))
        return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    if (T == 0) return ok();
    const bool need_cache = rot_dim > 0 && max_pos > 0;
    if ((Q > 0 && !q) || (K > 0 && !k)) return fail(MBT_ERR_NULL_POINTER, "q / k required");
    if (!pos) return fail(MBT_ERR_NULL_POINTER, "pos is required");
    if (need_cache && !cos_sin)
        return fail(MBT_ERR_NULL_POINTER, "cos_sin is required when rot_dim > 0");
    if ((Q > 0 && !aligned(q, eb)) || (K > 0 && !aligned(k, eb)) || !aligned(pos, 8) ||
        (need_cache && !aligned(cos_sin, 4)))
        return fail(MBT_ERR_ALIGN, "a pointer is not aligned to its element size");
    const Range qr{(const char*)(Q ? q : nullptr), q_bytes, "q"};
    const Range kr{(const char*)(K ? k : nullptr), k_bytes, "k"};
    const Range cs{(const char*)(need_cache ? cos_sin : nullptr), cs_bytes, "cos_sin"};
    const Range ps{(const char*)pos, T * 8, "pos"};
    if (overlap(qr, kr)) return fail(MBT_ERR_ALIAS, "q overlaps k");
    for (const Range* o : {&qr, &kr})
        for (const Range* i : {&cs, &ps}) {
            mbt_status st = check_alias(*o, *i, false);
            if (st != MBT_OK) return st;
        }
    mbt::RopeArgs a{q, k, cos_sin, max_pos, pos, Q, K, T, head_dim, rot_dim, layout, dtype};
    return hip_status(mbt::launch_rope(a, (hipStream_t)stream), "rope launch");
}

namespace {

mbt_status norm_common(const void* x, const void* residual, const void* w, int64_t T,
                       int32_t H, float eps, int32_t weight_offset, int32_t dtype,
                       int64_t* row_bytes) {
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (weight_offset != 0 && weight_offset != 1)
        return fail(MBT_ERR_BAD_ENUM, "weight_offset %d", weight_offset);
    if (T < 0 || H < 1 || H > kMaxRow)
        return fail(MBT_ERR_BAD_SHAPE, "T=%lld H=%d", (long long)T, H);
    if (!finite_nonneg(eps)) return fail(MBT_ERR_BAD_SCALAR, "eps must be finite and >= 0");
    const int eb = elt_bytes(dtype);
    const int64_t bytes = mul(mul(T, H), eb);
    if (bytes < 0) return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    *row_bytes = bytes;
    if (T == 0) return MBT_OK;
    if (!x) return fail(MBT_ERR_NULL_POINTER, "x is required");
    if (!w && weight_offset != 0)
        return fail(MBT_ERR_NULL_POINTER, "w is required with weight_offset 1");
    if (!aligned(x, eb) || (w && !aligned(w, eb)) || (residual && !aligned(residual, eb)))
        return fail(MBT_ERR_ALIGN, "a pointer is not aligned to its element size");
    const Range xr{(const char*)x, bytes, "x"};
    const Range rr{(const char*)residual, bytes, "residual"};
    const Range wr{(const char*)w, (int64_t)H * eb, "w"};
    if (overlap(xr, rr)) return fail(MBT_ERR_ALIAS, "residual overlaps x");
    if (overlap(wr, xr) || overlap(wr, rr)) return fail(MBT_ERR_ALIAS, "w overlaps x or residual");
    return MBT_OK;
}

}  // namespace

mbt_status mbt_fused_add_rmsnorm(void* x, void* residual, const void* w, int64_t T, int32_t H,
                                 float eps, int32_t weight_offset, int32_t dtype,
                                 void* stream) {
    int64_t bytes = 0;
    mbt_status st = norm_common(x, residual, w, T, H, eps, weight_offset, dtype, &bytes);
    if (st != MBT_OK) return st;
    if (T == 0) return ok();
    mbt::NormArgs a{};
    a.x = x; a.x_out = x; a.residual = residual; a.w = w; a.T = T; a.H = H; a.eps = eps;
    a.weight_offset = weight_offset; a.dtype = dtype; a.mode = mbt::kNormInPlace;
    return hip_status(mbt::launch_rmsnorm(a, (hipStream_t)stream), "fused_add_rmsnorm launch");
}

mbt_status mbt_fused_add_rmsnorm_fp8(const void* x, void* residual, const void* w, uint8_t* y,
                                     float inv_scale, int64_t T, int32_t H, float eps,
                                     int32_t weight_offset, int32_t dtype, void* stream) {
    int64_t bytes = 0;
    mbt_status st = norm_common(x, residual, w, T, H, eps, weight_offset, dtype, &bytes);
    if (st != MBT_OK) return st;
    if (!finite_pos(inv_scale)) return fail(MBT_ERR_BAD_SCALAR, "inv_scale must be finite and > 0");
    if (T == 0) return ok();
    if (!y) return fail(MBT_ERR_NULL_POINTER, "y is required");
    const int eb = elt_bytes(dtype);
    const Range yr{(const char*)y, T * (int64_t)H, "y"};
    for (const Range& in : {Range{(const char*)x, bytes, "x"},
                            Range{(const char*)residual, bytes, "residual"},
                            Range{(const char*)w, (int64_t)H * eb, "w"}}) {
        st = check_alias(yr, in, false);
        if (st != MBT_OK) return st;
    }
    mbt::NormArgs a{};
    a.x = x; a.residual = residual; a.w = w; a.y8 = y; a.inv_scale = inv_scale; a.T = T;
    a.H = H; a.eps = eps; a.weight_offset = weight_offset; a.dtype = dtype;
    a.mode = mbt::kNormFp8;
    return hip_status(mbt::launch_rmsnorm(a, (hipStream_t)stream),
                      "fused_add_rmsnorm_fp8 launch");
}

mbt_status mbt_fused_add_rmsnorm_amax(const void* x, const void* residual, const void* w,
                                      float* amax, int64_t T, int32_t H, float eps,
                                      int32_t weight_offset, int32_t dtype, void* stream) {
    int64_t bytes = 0;
    mbt_status st = norm_common(x, residual, w, T, H, eps, weight_offset, dtype, &bytes);
    if (st != MBT_OK) return st;
    if (T == 0) return ok();
    if (!amax) return fail(MBT_ERR_NULL_POINTER, "amax is required");
    if (!aligned(amax, 4)) return fail(MBT_ERR_ALIGN, "amax must be 4-byte aligned");
    const int eb = elt_bytes(dtype);
    const Range ar{(const char*)amax, 4, "amax"};
    for (const Range& in : {Range{(const char*)x, bytes, "x"},
                            Range{(const char*)residual, bytes, "residual"},
                            Range{(const char*)w, (int64_t)H * eb, "w"}}) {
        st = check_alias(ar, in, false);
        if (st != MBT_OK) return st;
    }
    mbt::NormArgs a{};
    a.x = x; a.residual = const_cast<void*>(residual); a.w = w; a.amax = amax; a.T = T;
    a.H = H; a.eps = eps; a.weight_offset = weight_offset; a.dtype = dtype;
    a.mode = mbt::kNormAmax;
    return hip_status(mbt::launch_rmsnorm(a, (hipStream_t)stream),
                      "fused_add_rmsnorm_amax launch");
}

namespace {

// Adaptive RMSNorm: the residual-norm checks with w = scale, plus shift
// (required) and gate (optional, needs a residual).  `outs` are the ranges
// the call writes besides residual / x.
mbt_status ada_common(const void* x, const void* residual, const void* gate, const void* scale,
                      const void* shift, int64_t T, int32_t H, float eps, int32_t dtype,
                      int64_t* bytes) {
    if (gate && !residual && T > 0)
        return fail(MBT_ERR_NULL_POINTER, "a gate needs a residual");
    if (T > 0 && !scale) return fail(MBT_ERR_NULL_POINTER, "scale is required");
    mbt_status st = norm_common(x, residual, scale, T, H, eps, 1, dtype, bytes);
    if (st != MBT_OK || T == 0) return st;
    if (!shift) return fail(MBT_ERR_NULL_POINTER, "shift is required");
    const int eb = elt_bytes(dtype);
    if (!aligned(shift, eb) || (gate && !aligned(gate, eb)))
        return fail(MBT_ERR_ALIGN, "a pointer is not aligned to its element size");
    const Range xr{(const char*)x, *bytes, "x"};
    const Range rr{(const char*)residual, *bytes, "residual"};
    for (const Range& v : {Range{(const char*)shift, (int64_t)H * eb, "shift"},
                           Range{(const char*)gate, (int64_t)H * eb, "gate"}})
        if (overlap(v, xr) || overlap(v, rr))
            return fail(MBT_ERR_ALIAS, "%s overlaps x or residual", v.name);
    return MBT_OK;
}

mbt_status ada_launch(mbt::NormArgs a, const void* gate, const void* shift, void* stream,
                      const char* what) {
    a.ada = true;
    a.gate = gate;
    a.shift = shift;
    a.weight_offset = 1;                      // w = scale: the weight path gives 1 + scale
    return hip_status(mbt::launch_rmsnorm(a, (hipStream_t)stream), what);
}

}  // namespace

mbt_status mbt_adarms(void* x, void* residual, const void* gate, const void* scale,
                      const void* shift, int64_t T, int32_t H, float eps, int32_t dtype,
                      void* stream) {
    int64_t bytes = 0;
    mbt_status st = ada_common(x, residual, gate, scale, shift, T, H, eps, dtype, &bytes);
    if (st != MBT_OK) return st;
    if (T == 0) return ok();
    mbt::NormArgs a{};
    a.x = x; a.x_out = x; a.residual = residual; a.w = scale; a.T = T; a.H = H; a.eps = eps;
    a.dtype = dtype; a.mode = mbt::kNormInPlace;
    return ada_launch(a, gate, shift, stream, "adarms launch");
}

mbt_status mbt_adarms_fp8(const void* x, void* residual, const void* gate, const void* scale,
                          const void* shift, uint8_t* y, float inv_scale, int64_t T, int32_t H,
                          float eps, int32_t dtype, void* stream) {
    int64_t bytes = 0;
    mbt_status st = ada_common(x, residual, gate, scale, shift, T, H, eps, dtype, &bytes);
    if (st != MBT_OK) return st;
    if (!finite_pos(inv_scale)) return fail(MBT_ERR_BAD_SCALAR, "inv_scale must be finite > 0");
    if (T == 0) return ok();
    if (!y) return fail(MBT_ERR_NULL_POINTER, "y is required");
    const int eb = elt_bytes(dtype);
    const Range yr{(const char*)y, mul(T, H), "y"};
    for (const Range& in : {Range{(const char*)x, bytes, "x"},
                            Range{(const char*)residual, bytes, "residual"},
                            Range{(const char*)scale, (int64_t)H * eb, "scale"},
                            Range{(const char*)shift, (int64_t)H * eb, "shift"},
                            Range{(const char*)gate, (int64_t)H * eb, "gate"}}) {
        st = check_alias(yr, in, false);
        if (st != MBT_OK) return st;
    }
    mbt::NormArgs a{};
    a.x = x; a.residual = residual; a.w = scale; a.y8 = y; a.inv_scale = inv_scale; a.T = T;
    a.H = H; a.eps = eps; a.dtype = dtype; a.mode = mbt::kNormFp8;
    return ada_launch(a, gate, shift, stream, "adarms_fp8 launch");
}

mbt_status mbt_adarms_amax(const void* x, const void* residual, const void* gate,
                           const void* scale, const void* shift, float* amax, int64_t T,
                           int32_t H, float eps, int32_t dtype, void* stream) {
    int64_t bytes = 0;
    mbt_status st = ada_common(x, residual, gate, scale, shift, T, H, eps, dtype, &bytes);
    if (st != MBT_OK) return st;
    if (T == 0) return ok();
    if (!amax) return fail(MBT_ERR_NULL_POINTER, "amax is required");
    if (!aligned(amax, 4)) return fail(MBT_ERR_ALIGN, "amax must be 4-byte aligned");
    const int eb = elt_bytes(dtype);
    const Range ar{(const char*)amax, 4, "amax"};
    for (const Range& in : {Range{(const char*)x, bytes, "x"},
                            Range{(const char*)residual, bytes, "residual"},
                            Range{(const char*)scale, (int64_t)H * eb, "scale"},
                            Range{(const char*)shift, (int64_t)H * eb, "shift"},
                            Range{(const char*)gate, (int64_t)H * eb, "gate"}}) {
        st = check_alias(ar, in, false);
        if (st != MBT_OK) return st;
    }
    mbt::NormArgs a{};
    a.x = x; a.residual = const_cast<void*>(residual); a.w = scale; a.amax = amax; a.T = T;
    a.H = H; a.eps = eps; a.dtype = dtype; a.mode = mbt::kNormAmax;
    return ada_launch(a, gate, shift, stream, "adarms_amax launch");
}

namespace {

mbt_status act_common(const void* gate_up, int64_t T, int32_t d, int32_t act, int32_t dtype,
                      int64_t* in_bytes) {
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (act != MBT_ACT_SILU && act != MBT_ACT_GELU_TANH)
        return fail(MBT_ERR_BAD_ENUM, "act %d", act);
    if (T < 0 || d < 1 || d > kMaxRow)
        return fail(MBT_ERR_BAD_SHAPE, "T=%lld d=%d", (long long)T, d);
    const int eb = elt_bytes(dtype);
    const int64_t bytes = mul(mul(T, 2 * (int64_t)d), eb);
    if (bytes < 0) return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    *in_bytes = bytes;
    if (T == 0) return MBT_OK;
    if (!gate_up) return fail(MBT_ERR_NULL_POINTER, "gate_up is required");
    if (!aligned(gate_up, eb)) return fail(MBT_ERR_ALIGN, "gate_up is not element aligned");
    return MBT_OK;
}

}  // namespace

mbt_status mbt_gated_act(const void* gate_up, void* out, int64_t T, int32_t d, int32_t act,
                         int32_t dtype, void* stream) {
    int64_t in_bytes = 0;
    mbt_status st = act_common(gate_up, T, d, act, dtype, &in_bytes);
    if (st != MBT_OK) return st;
    if (T == 0) return ok();
    if (!out) return fail(MBT_ERR_NULL_POINTER, "out is required");
    const int eb = elt_bytes(dtype);
    if (!aligned(out, eb)) return fail(MBT_ERR_ALIGN, "out is not element aligned");
    st = check_alias(Range{(const char*)out, T * (int64_t)d * eb, "out"},
                     Range{(const char*)gate_up, in_bytes, "gate_up"}, false);
    if (st != MBT_OK) return st;
    mbt::ActArgs a{};
    a.gate_up = gate_up; a.out = out; a.T = T; a.d = d; a.act = act; a.dtype = dtype;
    a.mode = mbt::kActDtype;
    return hip_status(mbt::launch_gated_act(a, (hipStream_t)stream), "gated_act launch");
}

mbt_status mbt_gated_act_fp8(const void* gate_up, uint8_t* out, float inv_scale, int64_t T,
                             int32_t d, int32_t act, int32_t dtype, void* stream) {
    int64_t in_bytes = 0;
    mbt_status st = act_common(gate_up, T, d, act, dtype, &in_bytes);
    if (st != MBT_OK) return st;
    if (!finite_pos(inv_scale)) return fail(MBT_ERR_BAD_SCALAR, "inv_scale must be finite and > 0");
    if (T == 0) return ok();
    if (!out) return fail(MBT_ERR_NULL_POINTER, "out is required");
    st = check_alias(Range{(const char*)out, T * (int64_t)d, "out"},
                     Range{(const char*)gate_up, in_bytes, "gate_up"}, false);
    if (st != MBT_OK) return st;
    mbt::ActArgs a{};
    a.gate_up = gate_up; a.out8 = out; a.inv_scale = inv_scale; a.T = T; a.d = d; a.act = act;
    a.dtype = dtype; a.mode = mbt::kActFp8;
    return hip_status(mbt::launch_gated_act(a, (hipStream_t)stream), "gated_act_fp8 launch");
}

mbt_status mbt_gated_act_amax(const void* gate_up, float* amax, int64_t T, int32_t d,
                              int32_t act, int32_t dtype, void* stream) {
    int64_t in_bytes = 0;
    mbt_status st = act_common(gate_up, T, d, act, dtype, &in_bytes);
    if (st != MBT_OK) return st;
    if (T == 0) return ok();
    if (!amax) return fail(MBT_ERR_NULL_POINTER, "amax is required");
    if (!aligned(amax, 4)) return fail(MBT_ERR_ALIGN, "amax must be 4-byte aligned");
    st = check_alias(Range{(const char*)amax, 4, "amax"},
                     Range{(const char*)gate_up, in_bytes, "gate_up"}, false);
    if (st != MBT_OK) return st;
    mbt::ActArgs a{};
    a.gate_up = gate_up; a.amax = amax; a.T = T; a.d = d; a.act = act; a.dtype = dtype;
    a.mode = mbt::kActAmax;
    return hip_status(mbt::launch_gated_act(a, (hipStream_t)stream), "gated_act_amax launch");
}

mbt_status mbt_quantize_fp8(const float* x, uint8_t* y, int64_t n, float inv_scale,
                            void* stream) {
    if (n < 0) return fail(MBT_ERR_BAD_SHAPE, "n=%lld", (long long)n);
    if (!finite_pos(inv_scale)) return fail(MBT_ERR_BAD_SCALAR, "inv_scale must be finite and > 0");
    if (mul(n, 4) < 0) return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    if (n == 0) return ok();
    if (!x || !y) return fail(MBT_ERR_NULL_POINTER, "x and y are required");
    if (!aligned(x, 4)) return fail(MBT_ERR_ALIGN, "x must be 4-byte aligned");
    mbt_status st = check_alias(Range{(const char*)y, n, "y"},
                                Range{(const char*)x, n * 4, "x"}, false);
    if (st != MBT_OK) return st;
    return hip_status(mbt::launch_quantize_fp8(x, y, n, inv_scale, (hipStream_t)stream),
                      "quantize_fp8 launch");
}

mbt_status mbt_stream_copy(const void* src, void* dst, int64_t nbytes, int32_t chunks_per_lane,
                           int32_t block_sync, void* stream) {
    // 2^40 bytes at one 16-byte chunk per lane is 2^28 blocks: every form launches
    if (nbytes < 0 || nbytes % 16 != 0 || nbytes > (INT64_C(1) << 40))
        return fail(MBT_ERR_BAD_SHAPE, "nbytes=%lld must be a multiple of 16 in [0, 2^40]",
                    (long long)nbytes);
    if (chunks_per_lane != 1 && chunks_per_lane != 2 && chunks_per_lane != 4 &&
        chunks_per_lane != 8)
        return fail(MBT_ERR_BAD_ENUM, "chunks_per_lane %d not 1, 2, 4 or 8", chunks_per_lane);
    if (block_sync != 0 && block_sync != 1)
        return fail(MBT_ERR_BAD_ENUM, "block_sync %d not 0 or 1", block_sync);
    if (nbytes == 0) return ok();
    if (!src || !dst) return fail(MBT_ERR_NULL_POINTER, "src and dst are required");
    if (!aligned(src, 16) || !aligned(dst, 16))
        return fail(MBT_ERR_ALIGN, "src and dst must be 16-byte aligned");
    if (overlap(Range{(const char*)src, nbytes, "src"}, Range{(const char*)dst, nbytes, "dst"}))
        return fail(MBT_ERR_ALIAS, "dst overlaps src");
    return hip_status(mbt::launch_stream_copy(src, dst, nbytes, chunks_per_lane,
                                              block_sync != 0, (hipStream_t)stream),
                      "stream_copy launch");
}

}  // extern "C"
