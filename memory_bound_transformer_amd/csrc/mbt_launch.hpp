// mbt_launch.hpp -- internal interface between the C-ABI layer (mbt_api.cpp)
// and the kernel launchers.  Arguments reaching a launcher are already
// validated; launchers only choose a kernel and a grid and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbt {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct QkArgs {
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
    int32_t head_dim, rot_dim;
    float eps;
    int32_t weight_offset, layout, dtype;
    // token strides in elements (dense: heads * head_dim)
    int64_t q_in_stride, k_in_stride, q_out_stride, k_out_stride;
    bool round_once;
    // key / value rows of token t go to row slot[t] of k_out / v_out when
    // slot is given (rows outside [0, n_slots) are not written)
    const int64_t* slot;
    int64_t n_slots;
    // value rows copied unchanged (NULL v_in: none)
    const void* v_in;
    void* v_out;
    int64_t v_in_stride, v_out_stride;
};

enum NormOut : int { kNormInPlace = 0, kNormFp8 = 1, kNormAmax = 2 };

struct NormArgs {
    const void* x;        // input rows
    void* x_out;          // normalised output (in-place form), else unused
    void* residual;       // may be NULL
    const void* w;
    uint8_t* y8;          // FP8 output
    float* amax;          // calibration output
    float inv_scale;
    int64_t T;
    int32_t H;
    float eps;
    int32_t weight_offset, dtype;
    int mode;             // NormOut
    // adaptive form (ada): w is the style scale (with weight_offset 1 it
    // gives 1 + scale), `shift` is added after it and `gate` multiplies x in
    // the residual sum (NULL: 1)
    bool ada;
    const void* gate;
    const void* shift;
};

enum ActOut : int { kActDtype = 0, kActFp8 = 1, kActAmax = 2 };

struct ActArgs {
    const void* gate_up;
    void* out;            // dtype output
    uint8_t* out8;        // FP8 output
    float* amax;
    float inv_scale;
    int64_t T;
    int32_t d;
    int32_t act, dtype;
    int mode;             // ActOut
};

struct RopeArgs {
    void* q;
    void* k;
    const float* cos_sin;
    int64_t max_pos;
    const int64_t* pos;
    int32_t Q, K;
    int64_t T;
    int32_t head_dim, rot_dim, layout, dtype;
};

hipError_t launch_qknorm_rope(const QkArgs& a, hipStream_t s);
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);
hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t s);
hipError_t launch_gated_act(const ActArgs& a, hipStream_t s);
hipError_t launch_quantize_fp8(const float* x, uint8_t* y, int64_t n, float inv_scale,
                               hipStream_t s);
// nbytes a multiple of 16, src and dst 16-byte aligned and disjoint;
// chunks (16-byte chunks per lane) 1, 2, 4 or 8; block_sync: a block's loads
// all land before any of its waves stores
hipError_t launch_stream_copy(const void* src, void* dst, int64_t nbytes, int chunks,
                              bool block_sync, hipStream_t s);

}  // namespace mbt
