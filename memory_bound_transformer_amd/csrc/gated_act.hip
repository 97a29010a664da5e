// gated_act.hip -- gated SiLU / GELU-tanh activation for gfx950, with a
// dtype output, a static-scale OCP e4m3fn output or a calibration amax; and
// the standalone static FP8 quantizer.
//
// Operation ("thox-edge-ops v2", section 5.1: each input row holds the gate
// projection followed by the up projection, [g || u]):
//   out[t][j] = R(act(g) * u),  g = gate_up[t][j],  u = gate_up[t][d + j],
//   SiLU(g) = g sigmoid(g),  GELU-tanh(g) = g sigmoid(2z),
//   z = sqrt(2/pi) (g + 0.044715 g^3)      (0.5 (1 + tanh z) = sigmoid(2z)).
// FP8 (FlashRT optimization details: GELU + gate + FP8 with packed 4 x FP8
// stores; quantize_fp8_static): out = E4M3FN((act(g) * u) * inv_scale).
//
// MI355X design: a pure stream.  Each lane moves one 16-byte chunk of g and
// the matching chunk of u (8 bf16 / fp16 or 4 fp32) and stores 16 bytes of
// output or 8 / 4 packed e4m3fn codes; a 256-thread block covers U chunks per
// lane of one token's row (or, where rows are whole 256-chunk groups, two
// groups that may lie in consecutive rows), so the token index is a scalar
// division per block, not per lane.  sigmoid is evaluated from e^-|x| so it
// can neither overflow nor cancel; 16-bit I/O takes e^-|x| from the hardware
// exp2 (with a rescale that keeps results below FLT_MIN), fp32 I/O from the
// full-accuracy expf.

#include "mbt_device.hpp"
#include "mbt_launch.hpp"

namespace mbt {
namespace {

struct ActParams {
    const void* gate_up;
    void* out;
    uint8_t* out8;
    float* amax;
    float inv_scale;
    int64_t T;
    int32_t d;
    int32_t chunks;           // d / Vec (vector kernel)
    int32_t blocks_per_row;   // vector kernel
};

// e^-a for a >= 0 on the hardware exp2 (v_exp_f32).  v_exp_f32 returns 0
// for results below the smallest normal float, yet e.g. SiLU(-90) =
// -90 e^-90 ~ -7e-38 is still a normal bf16; so the exponent is halved
// (exactly: the constant is -log2(e) / 2) and the result squared, which
// reaches the fp32 subnormals (e^-a for a up to 174 has its square root in
// the normal range) with no compare or select: two VALU slots beside the
// exp2, against five for a rescue of exponents below -126 by a select.
// Error: about twice v_exp_f32's (1 ulp) plus the square's rounding.
__device__ __forceinline__ float exp_neg(float a) {
    const float h = __builtin_amdgcn_exp2f(a * -0.72134752044448170f);
    return h * h;
}

template <int DT>
__device__ __forceinline__ float sigmoid(float x) {
    const float ax = fabsf(x);
    float e;
    if constexpr (DT == kF32) e = expf(-ax);           // full accuracy for fp32 I/O
    else e = exp_neg(ax);
    const float r = __builtin_amdgcn_rcpf(1.0f + e);   // v_rcp_f32, 1 ulp
    return x >= 0.0f ? r : e * r;
}

// GELU-tanh for 16-bit I/O.  z = sqrt(2/pi) g (1 + 0.044715 g^2) and the
// bracket is positive, so z has g's sign and |z| = |g| sqrt(2/pi) (1 +
// 0.044715 g^2): with k1 = -log2(e) sqrt(2/pi) and k3 = 0.044715 k1,
// h = 2^(|g| (k1 + k3 g^2)) = e^-|z| takes one multiply and one FMA
// beside the exp2 (against five instructions for z and one for its scaled
// magnitude), e^-|2z| = h^2 as in exp_neg, and the sign test reads g.  The
// exponent rounds differently from the oracle's z, by a few fp32 ulps, far
// inside the output's 16-bit rounding.
__device__ __forceinline__ float gelu_tanh16(float g) {
    constexpr float k1 = -1.44269504088896341f * 0.7978845608f;
    constexpr float k3 = k1 * 0.044715f;
    const float h = __builtin_amdgcn_exp2f(fabsf(g) * fmaf(k3, g * g, k1));
    const float e = h * h;
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return g * (g >= 0.0f ? r : e * r);
}

template <int DT, int ACT>
__device__ __forceinline__ float act_mul(float g, float u) {
    float a;
    if constexpr (ACT == 0) {
        a = g * sigmoid<DT>(g);
    } else if constexpr (DT == kF32) {
        const float z = 0.7978845608f * (g + 0.044715f * g * g * g);
        a = g * sigmoid<DT>(2.0f * z);
    } else {
        a = gelu_tanh16(g);
    }
    return a * u;
}

// Vector kernel: d a multiple of Vec<DT>; gate_up and out 16-byte aligned,
// out8 aligned to its 8- (16-bit) or 4-byte (fp32) store; a half row below
// 2^31 bytes.  All arguments come in one batch of scalar loads, and every
// access goes through a buffer resource over the token's gate half, up half
// or output row: chunks past d read zeros (act(0) * 0 = 0, so they leave
// amax alone) and their stores are dropped, with no branch around a load or
// store.
template <int DT, int ACT, int MODE, int U>
__global__ __launch_bounds__(256) void gated_vec(ActParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    asm volatile("" ::"s"(p.gate_up), "s"(p.d), "s"(p.blocks_per_row));
    if constexpr (MODE == kActDtype) asm volatile("" ::"s"(p.out));
    if constexpr (MODE == kActFp8) asm volatile("" ::"s"(p.out8), "s"(p.inv_scale));
    if constexpr (MODE == kActAmax) asm volatile("" ::"s"(p.amax));
    const uint32_t bpr = (uint32_t)p.blocks_per_row;
    const uint32_t tu = blockIdx.x / bpr;
    const int64_t t = tu;
    const int cb = (int)(blockIdx.x - tu * bpr);
    const uint32_t hb = (uint32_t)p.d * EB;                 // bytes of a half row
    const char* row = (const char*)p.gate_up + t * 2 * (int64_t)hb;
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc((void*)row, hb);
    const __amdgpu_buffer_rsrc_t ru = buf_rsrc((void*)(row + hb), hb);
    u32x4 gv[U], uv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t off = (uint32_t)((cb * U + k) * 256 + threadIdx.x) * 16u;
        gv[k] = buf_ld16_nt(rg, off);
        uv[k] = buf_ld16_nt(ru, off);
    }
    asm volatile("" ::: "memory");
    __amdgpu_buffer_rsrc_t ro = rg;
    if constexpr (MODE == kActDtype) ro = buf_rsrc((char*)p.out + t * (int64_t)hb, hb);
    if constexpr (MODE == kActFp8) ro = buf_rsrc(p.out8 + t * (int64_t)p.d, (uint32_t)p.d);
    float amax_acc = 0.0f;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t ch = (uint32_t)((cb * U + k) * 256 + threadIdx.x);
        float g[V], u[V], y[V];
        unpack<DT>(gv[k], g);
        unpack<DT>(uv[k], u);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = act_mul<DT, ACT>(g[i], u[i]);
        if constexpr (MODE == kActDtype) {
            buf_st16_nt(ro, ch * 16u, pack<DT>(y));
        } else if constexpr (MODE == kActFp8) {
            if constexpr (V == 8) {
                u32x2 c;
                c[0] = fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                             y[3] * p.inv_scale);
                c[1] = fp8x4(y[4] * p.inv_scale, y[5] * p.inv_scale, y[6] * p.inv_scale,
                             y[7] * p.inv_scale);
                buf_st8_nt(ro, ch * 8u, c);
            } else {
                buf_st4_nt(ro, ch * 4u, fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale,
                                              y[2] * p.inv_scale, y[3] * p.inv_scale));
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) amax_acc = fmaxf(amax_acc, fabsf(y[i]));
        }
    }
    if constexpr (MODE == kActAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if ((threadIdx.x & 63) == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Flat-group kernel: used where a row is a whole number gpr >= 2 of
// 256-chunk groups (d a multiple of 256 Vec) and lanes take two chunks.
// Block b takes groups 2b and 2b + 1 of the T gpr groups in row-major order,
// which may lie in consecutive rows, so every lane of every block has data;
// with one block per pair of groups of a row, an odd gpr left half of each
// row's last block without any (d = 10240 bf16: gpr = 5, a sixth of the
// waves' arithmetic spent on zeros).  A group past the last row gets empty
// buffer resources: its loads read zeros and its stores are dropped.
template <int DT, int ACT, int MODE>
__global__ __launch_bounds__(256) void gated_flat(ActParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    constexpr int U = 2;
    asm volatile("" ::"s"(p.gate_up), "s"(p.d), "s"(p.blocks_per_row), "s"(p.T));
    if constexpr (MODE == kActDtype) asm volatile("" ::"s"(p.out));
    if constexpr (MODE == kActFp8) asm volatile("" ::"s"(p.out8), "s"(p.inv_scale));
    if constexpr (MODE == kActAmax) asm volatile("" ::"s"(p.amax));
    const uint32_t gpr = (uint32_t)p.blocks_per_row;      // groups per row
    const uint32_t q0 = blockIdx.x * (uint32_t)U;
    const uint32_t t0 = q0 / gpr;
    const uint32_t c0 = q0 - t0 * gpr;
    const uint32_t hb = (uint32_t)p.d * EB;                 // bytes of a half row
    const int64_t ngroups = p.T * (int64_t)gpr;
    int64_t tk[U];
    uint32_t ck[U], live[U];
    u32x4 gv[U], uv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t c = c0 + (uint32_t)k;
        const uint32_t wrap = c >= gpr ? 1u : 0u;           // U <= gpr: one boundary at most
        tk[k] = (int64_t)(t0 + wrap);
        ck[k] = c - wrap * gpr;
        live[k] = (int64_t)q0 + k < ngroups ? 1u : 0u;
        const char* row = (const char*)p.gate_up + tk[k] * 2 * (int64_t)hb;
        const uint32_t off = (ck[k] * 256u + threadIdx.x) * 16u;
        gv[k] = buf_ld16_nt(buf_rsrc((void*)row, live[k] * hb), off);
        uv[k] = buf_ld16_nt(buf_rsrc((void*)(row + hb), live[k] * hb), off);
    }
    asm volatile("" ::: "memory");
    float amax_acc = 0.0f;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t ch = ck[k] * 256u + threadIdx.x;
        float g[V], u[V], y[V];
        unpack<DT>(gv[k], g);
        unpack<DT>(uv[k], u);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = act_mul<DT, ACT>(g[i], u[i]);
        if constexpr (MODE == kActDtype) {
            buf_st16_nt(buf_rsrc((char*)p.out + tk[k] * (int64_t)hb, live[k] * hb), ch * 16u,
                        pack<DT>(y));
        } else if constexpr (MODE == kActFp8) {
            const auto ro = buf_rsrc(p.out8 + tk[k] * (int64_t)p.d, live[k] * (uint32_t)p.d);
            if constexpr (V == 8) {
                u32x2 c;
                c[0] = fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                             y[3] * p.inv_scale);
                c[1] = fp8x4(y[4] * p.inv_scale, y[5] * p.inv_scale, y[6] * p.inv_scale,
                             y[7] * p.inv_scale);
                buf_st8_nt(ro, ch * 8u, c);
            } else {
                buf_st4_nt(ro, ch * 4u, fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale,
                                              y[2] * p.inv_scale, y[3] * p.inv_scale));
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) amax_acc = fmaxf(amax_acc, fabsf(y[i]));
        }
    }
    if constexpr (MODE == kActAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if ((threadIdx.x & 63) == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Half-chunk lanes (16-bit dtypes, few rows): each lane takes 8 bytes (four
// elements) of the gate and of the up half and a row twice the lanes.  With
// few rows most SIMDs are idle and a wave's arithmetic is its latency (each
// VALU instruction issues over 4 cycles; the activation's two quarter-rate
// transcendentals per element make it the longest of the three ops), so
// halving the elements per lane shortens every wave.  Each output is formed
// exactly as in the vector kernel.
template <int DT, int ACT, int MODE>
__global__ __launch_bounds__(256) void gated_half(ActParams p) {
    static_assert(DT != kF32, "16-bit dtypes");
    constexpr int EB = 2;
    asm volatile("" ::"s"(p.gate_up), "s"(p.d), "s"(p.blocks_per_row));
    if constexpr (MODE == kActDtype) asm volatile("" ::"s"(p.out));
    if constexpr (MODE == kActFp8) asm volatile("" ::"s"(p.out8), "s"(p.inv_scale));
    if constexpr (MODE == kActAmax) asm volatile("" ::"s"(p.amax));
    const uint32_t bpr = (uint32_t)p.blocks_per_row;
    const uint32_t tu = blockIdx.x / bpr;
    const int64_t t = tu;
    const uint32_t h8 = (blockIdx.x - tu * bpr) * 256u + threadIdx.x;   // 8-byte unit
    const uint32_t hb = (uint32_t)p.d * EB;
    const char* row = (const char*)p.gate_up + t * 2 * (int64_t)hb;
    const u32x2 gv = buf_ld8_nt(buf_rsrc((void*)row, hb), h8 * 8u);
    const u32x2 uv = buf_ld8_nt(buf_rsrc((void*)(row + hb), hb), h8 * 8u);
    asm volatile("" ::: "memory");
    float g[8], u[8], y[4];
    unpack<DT>(u32x4{gv[0], gv[1], 0u, 0u}, g);
    unpack<DT>(u32x4{uv[0], uv[1], 0u, 0u}, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = act_mul<DT, ACT>(g[i], u[i]);
    if constexpr (MODE == kActDtype) {
        const u32x2 o{pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3])};
        buf_st8_nt(buf_rsrc((char*)p.out + t * (int64_t)hb, hb), h8 * 8u, o);
    } else if constexpr (MODE == kActFp8) {
        buf_st4_nt(buf_rsrc(p.out8 + t * (int64_t)p.d, (uint32_t)p.d), h8 * 4u,
                   fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                         y[3] * p.inv_scale));
    } else {
        float amax_acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) amax_acc = fmaxf(amax_acc, fabsf(y[i]));
        amax_acc = seg_max<64>(amax_acc);
        if ((threadIdx.x & 63) == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Scalar kernel: any d, element-aligned pointers; 256 elements of one row
// per block.
template <int DT, int ACT, int MODE>
__global__ __launch_bounds__(256) void gated_scalar(ActParams p) {
    const uint32_t bpr = (uint32_t)p.blocks_per_row;
    const int64_t t = (int64_t)(blockIdx.x / bpr);
    const int j = (int)(blockIdx.x % bpr) * 256 + threadIdx.x;
    float amax_acc = 0.0f;
    if (j < p.d) {
        const int64_t gi = t * (2 * (int64_t)p.d) + j;
        const float y = act_mul<DT, ACT>(ld_elt<DT>(p.gate_up, gi),
                                         ld_elt<DT>(p.gate_up, gi + p.d));
        const int64_t o = t * (int64_t)p.d + j;
        if constexpr (MODE == kActDtype) st_elt<DT>(p.out, o, y);
        else if constexpr (MODE == kActFp8) p.out8[o] = fp8x1(y * p.inv_scale);
        else amax_acc = fabsf(y);
    }
    if constexpr (MODE == kActAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if ((threadIdx.x & 63) == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Launch-shape thresholds (compile-time constants, the measured best on
// MI355X): half-chunk lanes while the launch has at most kActHalfWaves
// waves (kActHalfWavesFp8 for FP8 output); two chunks per lane from
// kActU2Chunks chunks.
constexpr int64_t kActHalfWaves = 1024;
constexpr int64_t kActHalfWavesFp8 = 8192;
constexpr int64_t kActU2Chunks = 400000;

template <int DT, int ACT, int MODE>
hipError_t launch_mode(const ActArgs& a, hipStream_t s) {
    constexpr int V = Vec<DT>::n;
    ActParams p{};
    p.gate_up = a.gate_up; p.out = a.out; p.out8 = a.out8; p.amax = a.amax;
    p.inv_scale = a.inv_scale; p.T = a.T; p.d = a.d;
    bool vec = (a.d % V == 0) && aligned16(a.gate_up) &&
               (int64_t)a.d * EltBytes<DT>::n < (int64_t(1) << 31);
    if (MODE == kActDtype) vec = vec && aligned16(a.out);
    if (MODE == kActFp8)
        vec = vec && ((reinterpret_cast<uintptr_t>(a.out8) & (V == 8 ? 7u : 3u)) == 0);
    // Half-chunk lanes for 16-bit inputs at few rows.  Measured on MI355X,
    // SiLU, d = 10240, bf16 out: T = 1 / 16 cold 1.90 / 2.15 -> 1.83 / 2.04
    // us, warm (a graph of 32 calls on one buffer set) 2.10 / 2.15 -> 1.97 /
    // 2.00 us; past 1024 waves warm launches got slower.  FP8 output
    // converts and stores fewer bytes per element, so its arithmetic chain
    // is the longer share and half-chunk lanes pay up to 8192 waves (T = 204
    // at d = 10240): SiLU -> FP8 cold T = 1 / 64 / 128 / 200 2.00 / 2.54 /
    // 3.05 / 3.64 -> 1.91 / 2.37 / 2.91 / 3.52 us, warm T = 128 2.99 ->
    // 2.93 us; at 10240 waves (T = 256) 4.02 -> 4.62 us, so wider launches
    // keep the full chunk.
    if constexpr (DT != kF32) {
        const int64_t bpr = (2 * (int64_t)(a.d / V) + 255) / 256;     // 8-byte units
        const int64_t cap = MODE == kActFp8 ? kActHalfWavesFp8 : kActHalfWaves;
        if (vec && a.T * bpr * 4 <= cap && a.T * bpr <= 0x7FFFFFFFll) {
            p.chunks = a.d / V;
            p.blocks_per_row = (int32_t)bpr;
            hipLaunchKernelGGL((gated_half<DT, ACT, MODE>), dim3((uint32_t)(a.T * bpr)),
                               dim3(256), 0, s, p);
            return hipGetLastError();
        }
    }
    if (vec) {
        p.chunks = a.d / V;
        // Two chunks per lane only at prefill widths: at decode widths the
        // per-wave latency matters more than the per-wave overhead.
        const int U = (a.T * (int64_t)p.chunks >= kActU2Chunks) ? 2 : 1;
        // Whole 256-chunk groups per row: the flat-group kernel, measured
        // on MI355X at d = 10240 bf16 (five groups per row) against one
        // block per pair of a row's groups, together with the GELU-tanh
        // argument above: GELU -> FP8 T = 512 / 1024 / 2048 6.92 / 12.60 /
        // 21.74 -> 6.14 / 10.72 / 19.83 us, SiLU -> FP8 6.10 / 11.47 / 19.84
        // -> 5.99 / 10.35 / 19.43 us.  Three or four groups per block were
        // slower at T = 384 - 512 (GELU -> FP8 T = 512: 6.14 -> 6.56 / 6.77
        // us).
        if (U == 2 && p.chunks % 256 == 0 && p.chunks >= 512) {
            const int64_t groups = a.T * (int64_t)(p.chunks / 256);
            if (groups < (int64_t(1) << 32)) {
                p.blocks_per_row = p.chunks / 256;
                hipLaunchKernelGGL((gated_flat<DT, ACT, MODE>), dim3((uint32_t)((groups + 1) / 2)),
                                   dim3(256), 0, s, p);
                return hipGetLastError();
            }
        }
        p.blocks_per_row = (p.chunks + 256 * U - 1) / (256 * U);
        const int64_t blocks = a.T * (int64_t)p.blocks_per_row;
        if (blocks <= 0x7FFFFFFFll) {
            if (U == 2)
                hipLaunchKernelGGL((gated_vec<DT, ACT, MODE, 2>), dim3((uint32_t)blocks),
                                   dim3(256), 0, s, p);
            else
                hipLaunchKernelGGL((gated_vec<DT, ACT, MODE, 1>), dim3((uint32_t)blocks),
                                   dim3(256), 0, s, p);
            return hipGetLastError();
        }
    }
    p.blocks_per_row = (a.d + 255) / 256;
    const int64_t blocks = a.T * (int64_t)p.blocks_per_row;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gated_scalar<DT, ACT, MODE>), dim3((uint32_t)blocks), dim3(256), 0, s,
                       p);
    return hipGetLastError();
}

template <int DT, int ACT>
hipError_t launch_act(const ActArgs& a, hipStream_t s) {
    switch (a.mode) {
    case kActDtype: return launch_mode<DT, ACT, kActDtype>(a, s);
    case kActFp8: return launch_mode<DT, ACT, kActFp8>(a, s);
    default: return launch_mode<DT, ACT, kActAmax>(a, s);
    }
}

template <int DT>
hipError_t launch_dt(const ActArgs& a, hipStream_t s) {
    return a.act == 0 ? launch_act<DT, 0>(a, s) : launch_act<DT, 1>(a, s);
}

// Standalone quantizer: 4 fp32 values -> one packed u32 of codes per lane.
__global__ __launch_bounds__(256) void quantize_vec(const float* x, uint8_t* y, int64_t n4,
                                                    float inv_scale) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const u32x4 v = ld16_nt(x + 4 * i);
    st4_nt(y + 4 * i, fp8x4(__uint_as_float(v[0]) * inv_scale, __uint_as_float(v[1]) * inv_scale,
                            __uint_as_float(v[2]) * inv_scale, __uint_as_float(v[3]) * inv_scale));
}
__global__ __launch_bounds__(256) void quantize_scalar(const float* x, uint8_t* y, int64_t n,
                                                       float inv_scale) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = fp8x1(x[i] * inv_scale);
}

}  // namespace

hipError_t launch_gated_act(const ActArgs& a, hipStream_t s) {
    switch (a.dtype) {
    case kF32: return launch_dt<kF32>(a, s);
    case kF16: return launch_dt<kF16>(a, s);
    default: return launch_dt<kBF16>(a, s);
    }
}

hipError_t launch_quantize_fp8(const float* x, uint8_t* y, int64_t n, float inv_scale,
                               hipStream_t s) {
    if (aligned16(x) && (reinterpret_cast<uintptr_t>(y) & 3u) == 0) {
        const int64_t n4 = n / 4;
        if (n4 > 0) {
            const int64_t blocks = (n4 + 255) / 256;
            if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
            hipLaunchKernelGGL(quantize_vec, dim3((uint32_t)blocks), dim3(256), 0, s, x, y, n4,
                               inv_scale);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int64_t rest = n - 4 * n4;
        if (rest > 0)
            hipLaunchKernelGGL(quantize_scalar, dim3(1), dim3(256), 0, s, x + 4 * n4,
                               y + 4 * n4, rest, inv_scale);
        return hipGetLastError();
    }
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_scalar, dim3((uint32_t)blocks), dim3(256), 0, s, x, y, n,
                       inv_scale);
    return hipGetLastError();
}

}  // namespace mbt
