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
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (layout != MBT_ROPE_ROTATE_HALF && layout != MBT_ROPE_INTERLEAVED)
        return fail(MBT_ERR_BAD_ENUM, "layout %d", layout);
    if (weight_offset != 0 && weight_offset != 1)
        return fail(MBT_ERR_BAD_ENUM, "weight_offset %d", weight_offset);
    if (Q < 0 || K < 0 || Q + K < 1) return fail(MBT_ERR_BAD_SHAPE, "Q=%d K=%d", Q, K);
    if (T < 0) return fail(MBT_ERR_BAD_SHAPE, "T=%lld", (long long)T);
    if (head_dim < 1 || head_dim > 512)
        return fail(MBT_ERR_BAD_SHAPE, "head_dim %d not in [1, 512]", head_dim);
    if (rot_dim < 0 || rot_dim > head_dim || (rot_dim % 2) != 0)
        return fail(MBT_ERR_BAD_SHAPE, "rot_dim %d (head_dim %d)", rot_dim, head_dim);
    if (!finite_nonneg(eps)) return fail(MBT_ERR_BAD_SCALAR, "eps must be finite and >= 0");
    if (max_pos < 0) return fail(MBT_ERR_BAD_SCALAR, "max_pos %lld", (long long)max_pos);
    const int eb = elt_bytes(dtype);
    const int64_t q_bytes = mul(mul(mul(T, Q), head_dim), eb);
    const int64_t k_bytes = mul(mul(mul(T, K), head_dim), eb);
    const int64_t cs_bytes = mul(mul(max_pos, rot_dim), 4);
    if (q_bytes < 0 || k_bytes < 0 || cs_bytes < 0 || mul(T, Q + K) > (INT64_C(1) << 40))
        return fail(MBT_ERR_BAD_SHAPE, "tensor sizes overflow");
    if (T == 0) return ok();
    const bool need_cache = rot_dim > 0 && max_pos > 0;
    if (Q > 0 && (!q_in || !q_out || !w_q))
        return fail(MBT_ERR_NULL_POINTER, "q_in, q_out and w_q are required when Q > 0");
    if (K > 0 && (!k_in || !k_out || !w_k))
        return fail(MBT_ERR_NULL_POINTER, "k_in, k_out and w_k are required when K > 0");
    if (!pos) return fail(MBT_ERR_NULL_POINTER, "pos is required");
    if (need_cache && !cos_sin)
        return fail(MBT_ERR_NULL_POINTER, "cos_sin is required when rot_dim > 0");
    if ((Q > 0 && (!aligned(q_in, eb) || !aligned(q_out, eb) || !aligned(w_q, eb))) ||
        (K > 0 && (!aligned(k_in, eb) || !aligned(k_out, eb) || !aligned(w_k, eb))) ||
        !aligned(pos, 8) || (need_cache && !aligned(cos_sin, 4)))
        return fail(MBT_ERR_ALIGN, "a pointer is not aligned to its element size");
    const int64_t w_bytes = (int64_t)head_dim * eb;
    const Range qi{(const char*)(Q ? q_in : nullptr), q_bytes, "q_in"};
    const Range ki{(const char*)(K ? k_in : nullptr), k_bytes, "k_in"};
    const Range qo{(const char*)(Q ? q_out : nullptr), q_bytes, "q_out"};
    const Range ko{(const char*)(K ? k_out : nullptr), k_bytes, "k_out"};
    const Range wq{(const char*)(Q ? w_q : nullptr), w_bytes, "w_q"};
    const Range wk{(const char*)(K ? w_k : nullptr), w_bytes, "w_k"};
    const Range cs{(const char*)(need_cache ? cos_sin : nullptr), cs_bytes, "cos_sin"};
    const Range ps{(const char*)pos, T * 8, "pos"};
    const Range* ins[] = {&qi, &ki, &wq, &wk, &cs, &ps};
    for (const Range* o : {&qo, &ko}) {
        for (const Range* i : ins) {
            const bool same_ok = (o == &qo && i == &qi) || (o == &ko && i == &ki);
            mbt_status st = check_alias(*o, *i, same_ok);
            if (st != MBT_OK) return st;
        }
    }
    if (overlap(qo, ko)) return fail(MBT_ERR_ALIAS, "q_out overlaps k_out");

    mbt::QkArgs a{q_in, k_in, q_out, k_out, w_q, w_k, cos_sin, max_pos, pos, Q, K, T,
                  head_dim, rot_dim, eps, weight_offset, layout, dtype};
    return hip_status(mbt::launch_qknorm_rope(a, (hipStream_t)stream), "qknorm_rope launch");
}

mbt_status mbt_rope(void* q, void* k, const float* cos_sin, int64_t max_pos, const int64_t* pos,
                    int32_t Q, int32_t K, int64_t T, int32_t head_dim, int32_t rot_dim,
                    int32_t layout, int32_t dtype, void* stream) {
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (layout != MBT_ROPE_ROTATE_HALF && layout != MBT_ROPE_INTERLEAVED)
        return fail(MBT_ERR_BAD_ENUM, "layout %d", layout);
    if (Q < 0 || K < 0 || Q + K < 1) return fail(MBT_ERR_BAD_SHAPE, "Q=%d K=%d", Q, K);
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
    if (T < 0 || H < 1) return fail(MBT_ERR_BAD_SHAPE, "T=%lld H=%d", (long long)T, H);
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

mbt_status act_common(const void* gate_up, int64_t T, int32_t d, int32_t act, int32_t dtype,
                      int64_t* in_bytes) {
    if (!valid_dtype(dtype)) return fail(MBT_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (act != MBT_ACT_SILU && act != MBT_ACT_GELU_TANH)
        return fail(MBT_ERR_BAD_ENUM, "act %d", act);
    if (T < 0 || d < 1) return fail(MBT_ERR_BAD_SHAPE, "T=%lld d=%d", (long long)T, d);
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

}  // extern "C"
