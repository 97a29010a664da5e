// mbt_device.hpp -- device-side building blocks shared by the libmbt kernels
// (gfx950 / CDNA4, wave64).
//
//  * element codecs for fp32 / fp16 / bf16 and the OCP e4m3fn epilogue;
//  * 16-byte vector loads and stores (global_load/store_dwordx4);
//  * DPP and cross-row reductions over 4..64-lane segments of a wavefront.
//
// Numerics follow the contract of "thox-edge-ops v2" (section 3, R1): every
// input decodes exactly to fp32, arithmetic is fp32, and each output is
// rounded once to nearest-even by the hardware conversions
// (v_cvt_pk_bf16_f32, v_cvt_pk_f16_f32, v_cvt_pk_fp8_f32), which honour the
// default round-to-nearest-even mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbt {

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Elements carried by one 16-byte vector.
template <int DT> struct Vec { static constexpr int n = (DT == kF32) ? 4 : 8; };
template <int DT> struct EltBytes { static constexpr int n = (DT == kF32) ? 4 : 2; };

// ---- 16-byte global memory access -----------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming (nontemporal) forms for tensors each launch touches exactly
// once: the loads and stores carry the nt hint, so the lines neither evict
// reused data (weights, rotary rows) from L2 / Infinity Cache nor wait there.
// Measured on MI355X: a cold 59 MB copy runs at 5.4 TB/s with the hint and
// 4.6 TB/s without.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
// Raw buffer resource over [base, base + bytes): the hardware drops stores
// at offsets outside it (the buffer range check), so lanes past the end of
// a partial wave need no branch.  Word 3 is the gfx9-family format word
// (32-bit data).  base and bytes must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
// 16-byte store through a buffer resource (default cache policy).
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
// 16-byte store through a buffer resource with the nontemporal policy (the
// cache-policy operand's nt bit, kept by every IR pass, unlike the
// nontemporal metadata of a plain store).
__device__ __forceinline__ void buf_st16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 2);
}
// 16-byte loads through a buffer resource: offsets outside the range read
// zeros (the same range check), so a partial wave needs no branch around
// its loads either.  Default and nontemporal policies.
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}
// 8-byte loads through a buffer resource (same range rule).
__device__ __forceinline__ u32x2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_ld8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 2);
}
// 8- and 4-byte nontemporal stores through a buffer resource (packed FP8).
__device__ __forceinline__ void buf_st8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 2);
}
__device__ __forceinline__ void buf_st4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 2);
}
__device__ __forceinline__ void st8_nt(void* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st4_nt(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ---- codecs ----------------------------------------------------------------

// Decode the 16-byte vector `v` (Vec<DT>::n elements) to fp32, exactly.
template <int DT>
__device__ __forceinline__ void unpack(const u32x4 v, float* f) {
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    } else if constexpr (DT == kBF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // copy the element out first: a bit_cast applied directly to the
            // vector-element expression v[i] reads element 0 for every i
            const uint32_t w = v[i];
            const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        }
    }
}

// An fp32 value the compiler must treat as already rounded to fp32.  The
// AMDGPU backend otherwise folds an fp32 product followed by a narrowing to
// fp16 into one v_fma_mixlo_f16, which rounds the exact product once, straight
// to fp16, instead of to fp32 and then to fp16 (and turns -0 into +0); even
// -ffp-contract=off does not stop that fold.  The empty asm costs nothing.
__device__ __forceinline__ float as_f32(float v) {
    asm("" : "+v"(v));
    return v;
}
__device__ __forceinline__ _Float16 to_f16(float v) { return (_Float16)as_f32(v); }

// Round two fp32 values to a packed pair of 16-bit elements (RNE).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (DT == kBF16) {
        bf16x2_t v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2_t v = {to_f16(a), to_f16(b)};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// Round Vec<DT>::n fp32 values to one 16-byte vector of DT.
template <int DT>
__device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
    }
    return v;
}

// 16 bytes of the value 1.0 in DT (the weight vector of a norm without one).
template <int DT>
__device__ __forceinline__ u32x4 ones16() {
    constexpr uint32_t one = DT == kF32 ? 0x3F800000u : DT == kBF16 ? 0x3F803F80u : 0x3C003C00u;
    return u32x4{one, one, one, one};
}

// Scalar element access for the unaligned / odd-width kernels.
template <int DT>
__device__ __forceinline__ float ld_elt(const void* p, int64_t i) {
    if constexpr (DT == kF32) {
        return reinterpret_cast<const float*>(p)[i];
    } else if constexpr (DT == kBF16) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
    } else {
        return (float)reinterpret_cast<const _Float16*>(p)[i];
    }
}
template <int DT>
__device__ __forceinline__ void st_elt(void* p, int64_t i, float v) {
    if constexpr (DT == kF32) {
        reinterpret_cast<float*>(p)[i] = v;
    } else if constexpr (DT == kBF16) {
        reinterpret_cast<__bf16*>(p)[i] = (__bf16)v;
    } else {
        reinterpret_cast<_Float16*>(p)[i] = to_f16(v);
    }
}
// R(v) read back as fp32: the value a later step of a fused op consumes.
template <int DT>
__device__ __forceinline__ float round_trip(float v) {
    if constexpr (DT == kF32) {
        return v;
    } else if constexpr (DT == kBF16) {
        return (float)(__bf16)v;
    } else {
        return (float)to_f16(v);
    }
}

// OCP e4m3fn with saturation: +-inf and |v| > 448 clamp to +-448, NaN stays
// NaN; the hardware conversion then rounds to nearest-even (subnormals
// included).  Two values -> 16 bits; `hi` selects the upper half of `old`.
__device__ __forceinline__ float fp8_clamp(float v) {
    // IEEE 754-2019 minimum / maximum propagate a NaN (gfx950's
    // v_minimum3_f32 / v_maximum3_f32): two instructions, against a v_med3
    // (which does not return a NaN operand) plus a compare and a select
    return __builtin_elementwise_maximum(__builtin_elementwise_minimum(v, 448.0f), -448.0f);
}
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(c), fp8_clamp(d), w, true);
    return (uint32_t)w;
}
__device__ __forceinline__ uint8_t fp8x1(float a) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(a), 0, false);
    return (uint8_t)(w & 0xff);
}

// ---- reductions ------------------------------------------------------------

// DPP controls (GCN / CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <- 7 - i (in 8)
constexpr int kDppMirror = 0x140;     // row_mirror: lane i <- 15 - i (in 16)
constexpr int kDppQuadEven = 0xA0;    // quad_perm [0,0,2,2]: odd lanes take the even lane

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Cross-row exchanges on gfx950's VALU lane swaps (no LDS traffic):
// v_permlane16_swap on (v, v) leaves rows (r0, r0, r2, r2) in the first
// result and (r1, r1, r3, r3) in the second; v_permlane32_swap on (v, v)
// leaves (lo, lo) and (hi, hi).  Adding the two halves in that fixed order
// gives every lane of the 32- / 64-lane group the same bits.
__device__ __forceinline__ float xrow16_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xrow32_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xrow16_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow32_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned segments of SEG lanes (SEG in 4, 8, 16, 32, 64); every lane
// of a segment receives the segment's total.  Within a 16-lane DPP row the
// steps are xor-1, xor-2 (quad permutes) and the half / full row mirrors,
// which act as xor-4 / xor-8 once each quad / half-row already holds one
// value; wider segments add across rows with the lane swaps above.
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
    static_assert(SEG == 4 || SEG == 8 || SEG == 16 || SEG == 32 || SEG == 64, "segment");
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    if constexpr (SEG >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (SEG >= 16) v += dpp<kDppMirror>(v);
    if constexpr (SEG >= 32) v = xrow16_sum(v);
    if constexpr (SEG >= 64) v = xrow32_sum(v);
    return v;
}

template <int SEG>
__device__ __forceinline__ float seg_max(float v) {
    v = fmaxf(v, dpp<kDppQuadXor1>(v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v));
    if constexpr (SEG >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if constexpr (SEG >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    if constexpr (SEG >= 32) v = xrow16_max(v);
    if constexpr (SEG >= 64) v = xrow32_max(v);
    return v;
}

// ---- rotate-half partner exchange -----------------------------------------
//
// A row's chunk j (j < hv) pairs with chunk j + hv, hv = rot/2 / Vec.  With
// chunks in natural lane order the partner sits hv lanes away, so one
// ds_bpermute per dword (a lane permute through the LDS crossbar; no LDS
// memory is touched) fetches it for every hv with a single straight-line
// path.  A switch over per-hv DPP shifts was measured slower at decode
// widths: the jump into cold code costs more than the permute.  Every lane of
// the wave must execute this call; `is_a` marks the lanes holding the first
// half, and the result of lanes outside the rotated span is unused.
__device__ __forceinline__ u32x4 rot_partner(u32x4 v, int hv, bool is_a) {
    const int lane = (int)__lane_id();
    const int src = ((lane + (is_a ? hv : -hv)) & (kWave - 1)) << 2;   // byte index
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v[d]);
    return r;
}

// Rotation of one pair exactly as the operation is written: two rounded
// products and one rounded sum, never contracted into an FMA, so every
// route (fused prologue, standalone rotation) rounds identically.
__device__ __forceinline__ float rot_mac(float own, float c, float other, float s) {
#pragma clang fp contract(off)
    const float p = own * c;
    const float q = other * s;
    return p + q;
}

// Sum of squares of one 16-byte chunk, as an explicit FMA chain in element
// order.  Every kernel forms a row's sum the same way -- per-chunk chains,
// then a balanced tree over the chunk index (DPP and lane swaps in a wave,
// chunk groups combined pairwise) -- so the result does not depend on the
// launch shape, the alignment or which entry point computed it.
template <int DT>
__device__ __forceinline__ float chunk_sumsq(const float* f) {
    constexpr int V = Vec<DT>::n;
    float p = f[0] * f[0];
#pragma unroll
    for (int i = 1; i < V; ++i) p = __builtin_fmaf(f[i], f[i], p);
    return p;
}

// inv = 1 / sqrt(ss / n + eps) with the same rounding everywhere.
__device__ __forceinline__ float inv_rms(float ss, float inv_n, float eps) {
    return __builtin_amdgcn_rsqf(__builtin_fmaf(ss, inv_n, eps));
}

// Wave-uniform value as a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Fold a non-negative float into a device-wide maximum (bit patterns of
// non-negative floats order like the integers).
__device__ __forceinline__ void atomic_max_nonneg(float* dst, float v) {
    atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(v));
}

// 1 / sqrt(m) on the hardware reciprocal square root (about 1 ulp).
__device__ __forceinline__ float rsqrt_hw(float m) { return __builtin_amdgcn_rsqf(m); }

}  // namespace mbt
