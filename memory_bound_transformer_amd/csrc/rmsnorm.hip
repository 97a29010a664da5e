// rmsnorm.hip -- fused residual-add RMSNorm for gfx950, with an in-place
// dtype output, a static-scale OCP e4m3fn output, or a calibration amax.
//
// Operation ("thox-edge-ops v2", section 5.1: one kernel stores the sum back
// into the residual stream and normalises that rounded sum; section 3, R1:
// the stored sum equals an eager elementwise add bit for bit):
//   s = R(x + r);  r <- s;  x <- R((s * inv) * (w + delta)),
//   inv = 1 / sqrt(mean(s^2) + eps).
// Without a weight (w == NULL, delta 0; FlashRT optimization details, weight
// folding) x <- R(s * inv): the weight vector becomes a register constant of
// ones, so no weight is loaded and the multiply by exactly 1 changes nothing.
// Adaptive form (ADA; FlashRT's fused_adarms / gate_res_adarms kernels, with
// a style vector of per-channel scale, shift and gate): s = R(r + g * x),
// and the output value is (s * inv) * (1 + scale) + shift -- the weight path
// with w = scale and delta = 1, plus one add.
// FP8 epilogue (FlashRT optimization details, fused kernel table and static
// FP8 calibration): y = E4M3FN(((s * inv) * (w + delta)) * inv_scale) with x
// left unchanged; the calibration pass instead folds max |(s*inv)*(w+delta)|
// into a device scalar and writes nothing else.
//
// MI355X design: the row stays in registers from load to store (the single
// read pass the FlashRT notes credit for their norm speed-up), so HBM sees
// exactly one read of x, r, w and one write of r and the output.
//
//  * Rows of at most 64 16-byte chunks (e.g. a 256-wide head, or H <= 512
//    bf16) are G-lane segments of a wave, several rows per wave, one chunk
//    per lane: no barrier.
//  * Wider rows are spread over WPR waves of NCH chunks per lane (one chunk
//    per lane at decode widths, measured best); each 64-chunk group reduces
//    inside a wave with DPP and the group sums combine through LDS.  16-bit
//    rows of up to 256 chunks take half a chunk per lane up to 4096 waves
//    (twice the waves, half the arithmetic per wave, the same bits).
//  * The sum of squares is the same fixed tree in every kernel: an FMA chain
//    inside each chunk, then a balanced tree over the chunk index padded with
//    zeros to a power of two.  The result therefore does not depend on the
//    launch shape or the alignment, and a row normalised here equals the
//    fused QK-norm prologue's normalisation of the same head bit for bit.
//  * Odd widths and unaligned pointers take a two-pass scalar kernel with
//    the same tree.

#include "mbt_device.hpp"
#include "mbt_launch.hpp"

namespace mbt {
namespace {

struct NormParams {
    const void* x;
    void* x_out;
    void* residual;
    const void* w;
    uint8_t* y8;
    float* amax;
    float inv_scale;
    int64_t T;
    int32_t H;
    float eps, inv_H, delta;
    int32_t wpr;   // wide kernel: waves per row
    int32_t rpb;   // wide kernel: rows per block
    int32_t wsh;   // wide kernel: wave -> row in block is wave >> wsh
    const void* gate;    // adaptive form: residual gate (NULL: 1)
    const void* shift;   // adaptive form: added after the scale
};

template <int N>
__device__ __forceinline__ float fixed_tree(float* g) {
#pragma unroll
    for (int w = 1; w < N; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) g[i] += g[i + w];
    return g[0];
}
__device__ __forceinline__ float group_tree(float* g, int n) {
    for (int w = 1; w < n; w <<= 1)
        for (int i = 0; i + w < n; i += 2 * w) g[i] += g[i + w];
    return g[0];
}

// s = R(x + r) for one chunk (fp32 add of the decoded operands, one rounding),
// returned packed; x alone without a residual.  With a gate (adaptive form)
// s = R(r + g * x), the product rounded to fp32 first.
// s = R(x + r) (with the gate: R(g * x + r)), formed with no branch, and x
// itself selected when there is no residual (x + 0 would turn -0 into +0).
template <int DT, bool GATED>
__device__ __forceinline__ u32x4 residual_sum(u32x4 xv, u32x4 rv, u32x4 gv, bool has_res) {
    constexpr int V = Vec<DT>::n;
    float a[V], b[V];
    unpack<DT>(xv, a);
    unpack<DT>(rv, b);
    if constexpr (GATED) {
        float g[V];
        unpack<DT>(gv, g);
#pragma unroll
        for (int i = 0; i < V; ++i) a[i] = g[i] * a[i];
    }
#pragma unroll
    for (int i = 0; i < V; ++i) a[i] += b[i];
    const u32x4 sv = pack<DT>(a);
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = has_res ? sv[d] : xv[d];
    return out;
}

// Rows of at most G chunks (G in 4..64): G-lane segments, 64 / G rows per wave,
// four waves per block, one chunk per lane.  As in the wide kernel below,
// every access goes through a buffer resource over the wave's rows (its rows
// below T), and a lane past the row's last chunk takes an offset outside
// every range: it reads zeros and its stores are dropped, with no branch;
// the arguments come in one batch of scalar loads.
template <int DT, int G, int MODE, bool ADA>
__global__ __launch_bounds__(256) void rmsnorm_small(NormParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    constexpr int RPW = kWave / G;
    asm volatile("" ::"s"(p.x), "s"(p.residual), "s"(p.w), "s"(p.T), "s"(p.H), "s"(p.eps),
                 "s"(p.inv_H), "s"(p.delta));
    if constexpr (MODE == kNormInPlace) asm volatile("" ::"s"(p.x_out));
    if constexpr (MODE == kNormFp8) asm volatile("" ::"s"(p.y8), "s"(p.inv_scale));
    if constexpr (MODE == kNormAmax) asm volatile("" ::"s"(p.amax));
    if constexpr (ADA) asm volatile("" ::"s"(p.gate), "s"(p.shift));
    const int lane = threadIdx.x & 63;
    const int j = lane % G;
    const int64_t row0 = (int64_t)uniform((int)(blockIdx.x * 4u + (threadIdx.x >> 6))) * RPW;
    const int64_t row = row0 + lane / G;
    const int chunks = p.H / V;
    const bool have = row < p.T && j < chunks;
    const bool has_res = p.residual != nullptr;
    const int64_t nr = p.T - row0 < RPW ? (p.T - row0 > 0 ? p.T - row0 : 0) : RPW;
    const uint32_t hb = (uint32_t)p.H * EB;
    const uint32_t wb = (uint32_t)nr * hb;                 // bytes of the wave's rows
    const int64_t base = row0 * (int64_t)hb;
    const uint32_t off = j < chunks ? (uint32_t)((lane / G) * hb + j * 16) : 0xFFFFFFF0u;
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc((char*)p.x + base, wb);
    const __amdgpu_buffer_rsrc_t rr =
        buf_rsrc(has_res ? (char*)p.residual + base : (char*)p.x, has_res ? wb : 0u);
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc((void*)p.w, p.w ? hb : 0u);
    const u32x4 xv = buf_ld16_nt(rx, off);
    const u32x4 rv = buf_ld16_nt(rr, off);
    u32x4 wv = buf_ld16(rw, (uint32_t)j * 16u), gv = ones16<DT>();
    if constexpr (ADA) gv = buf_ld16(buf_rsrc((void*)p.gate, p.gate ? hb : 0u), (uint32_t)j * 16u);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < 4; ++d) wv[d] = p.w ? wv[d] : ones16<DT>()[d];
    if constexpr (ADA)
#pragma unroll
        for (int d = 0; d < 4; ++d) gv[d] = p.gate ? gv[d] : ones16<DT>()[d];
    const u32x4 sv = residual_sum<DT, ADA>(xv, rv, gv, has_res);
    float s[V];
    unpack<DT>(sv, s);
    const float ss = seg_sum<G>(chunk_sumsq<DT>(s));        // lanes past the row add 0
    const float inv = inv_rms(ss, p.inv_H, p.eps);
    // (no residual: rr has range 0 and the store is dropped)
    if constexpr (MODE != kNormAmax) buf_st16_nt(rr, off, sv);
    float wf[V], y[V];
    unpack<DT>(wv, wf);
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = (s[i] * inv) * (wf[i] + p.delta);
    if constexpr (ADA) {
        float sh[V];
        unpack<DT>(buf_ld16(buf_rsrc((void*)p.shift, hb), (uint32_t)j * 16u), sh);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] += sh[i];
    }
    float amax_acc = 0.0f;
    if constexpr (MODE == kNormInPlace) {
        buf_st16_nt(buf_rsrc((char*)p.x_out + base, wb), off, pack<DT>(y));
    } else if constexpr (MODE == kNormFp8) {
        const __amdgpu_buffer_rsrc_t ry = buf_rsrc(p.y8 + row0 * (int64_t)p.H, (uint32_t)nr * (uint32_t)p.H);
        const uint32_t o8 = j < chunks ? (uint32_t)((lane / G) * p.H + j * V) : 0xFFFFFFF0u;
        if constexpr (V == 8) {
            u32x2 c;
            c[0] = fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                         y[3] * p.inv_scale);
            c[1] = fp8x4(y[4] * p.inv_scale, y[5] * p.inv_scale, y[6] * p.inv_scale,
                         y[7] * p.inv_scale);
            buf_st8_nt(ry, o8, c);
        } else {
            buf_st4_nt(ry, o8, fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale,
                                     y[2] * p.inv_scale, y[3] * p.inv_scale));
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) amax_acc = fmaxf(amax_acc, have ? fabsf(y[i]) : 0.0f);
        amax_acc = seg_max<64>(amax_acc);
        if (lane == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Rows of more than 64 chunks: WPR waves per row (RPB rows per block when
// WPR divides 4), NCH chunks per lane.  Chunk ch = k * 64 * WPR + wave * 64
// + lane, so chunk group g = k * WPR + wave holds 64 consecutive chunks.
//
// Every access goes through a buffer resource over the wave's row (range 0
// for a row past T, and for a residual that is NULL): chunks past the row
// read zeros and their stores are dropped, so no load or store sits behind
// a branch and the loads go out back to back.  All arguments come in one
// batch of scalar loads, and the wave's row in the block is a shift, not a
// division.  Measured on MI355X, cold, bf16, against the branched form with
// two argument rounds: residual norm H = 2560 T = 1 / 128 / 512 2.37 / 2.86
// / 3.69 -> 2.09 / 2.60 / 3.40 us; norm -> FP8 H = 2048 T = 128 / 2048 2.75
// / 6.67 -> 2.62 / 6.00 us.  Storing the residual sum before the reduction
// (to overlap the barrier) gained nothing at one chunk per lane and cost 17 %
// at four (T = 2048), so it is stored with the output.
constexpr int kMaxNch = 6;
constexpr int kMaxGroups = kMaxNch * 16;

template <int DT, int NCH, int MODE, bool ADA>
__global__ __launch_bounds__(1024) void rmsnorm_vec(NormParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    __shared__ float gsum[4][kMaxGroups];
    asm volatile("" ::"s"(p.x), "s"(p.residual), "s"(p.w), "s"(p.T), "s"(p.H), "s"(p.eps),
                 "s"(p.inv_H), "s"(p.delta), "s"(p.wpr), "s"(p.rpb), "s"(p.wsh));
    if constexpr (MODE == kNormInPlace) asm volatile("" ::"s"(p.x_out));
    if constexpr (MODE == kNormFp8) asm volatile("" ::"s"(p.y8), "s"(p.inv_scale));
    if constexpr (MODE == kNormAmax) asm volatile("" ::"s"(p.amax));
    if constexpr (ADA) asm volatile("" ::"s"(p.gate), "s"(p.shift));
    const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const int wpr = p.wpr;
    const int rib = wave >> p.wsh, wir = wave - rib * wpr;   // row in block, wave in row
    const int64_t row = (int64_t)blockIdx.x * p.rpb + rib;
    const bool live = row < p.T;                               // wave-uniform
    const int chunks = p.H / V;
    const int ngroups = (chunks + kWave - 1) / kWave;
    const int stride = kWave * wpr;
    const bool has_res = p.residual != nullptr;
    const uint32_t hb = (uint32_t)p.H * EB;                   // bytes of a row
    const uint32_t rb = live ? hb : 0u;
    const int64_t ro = live ? row * (int64_t)hb : 0;
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc((char*)p.x + ro, rb);
    const __amdgpu_buffer_rsrc_t rr =
        buf_rsrc(has_res ? (char*)p.residual + ro : (char*)p.x, has_res ? rb : 0u);
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc((void*)p.w, p.w ? hb : 0u);
    __amdgpu_buffer_rsrc_t rg = rw;
    if constexpr (ADA) rg = buf_rsrc((void*)p.gate, p.gate ? hb : 0u);

    // Every load of the row (x, residual, weight, gate) before any math.
    u32x4 xv[NCH], rv[NCH], wv[NCH], gv[ADA ? NCH : 1];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const uint32_t off = (uint32_t)(k * stride + wir * kWave + lane) * 16u;
        xv[k] = buf_ld16_nt(rx, off);
        rv[k] = buf_ld16_nt(rr, off);
        wv[k] = buf_ld16(rw, off);
        if constexpr (ADA) gv[k] = buf_ld16(rg, off);
    }
    asm volatile("" ::: "memory");
    const bool has_w = p.w != nullptr;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int d = 0; d < 4; ++d) wv[k][d] = has_w ? wv[k][d] : ones16<DT>()[d];
    if constexpr (ADA) {
        const bool has_g = p.gate != nullptr;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int d = 0; d < 4; ++d) gv[k][d] = has_g ? gv[k][d] : ones16<DT>()[d];
    }

    // s = R(x + r); group sums: chunk chains, then the 64-lane tree of each
    // group (chunks past the row are zeros)
    float gs[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        xv[k] = residual_sum<DT, ADA>(xv[k], rv[k], gv[ADA ? k : 0], has_res);   // s
        float s[V];
        unpack<DT>(xv[k], s);
        gs[k] = seg_sum<64>(chunk_sumsq<DT>(s));
    }
    float ss;
    if (wpr == 1) {
        ss = fixed_tree<NCH>(gs);                      // groups past the row are 0
    } else {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int g = k * wpr + wir;
            if (lane == 0 && g < ngroups) gsum[rib][g] = gs[k];
        }
        __syncthreads();
        // group g in lane g (and g - 64): the 64-lane tree is the balanced
        // tree over the padded group slots
        const float lo = lane < ngroups ? gsum[rib][lane] : 0.0f;
        const float hi = lane + kWave < ngroups ? gsum[rib][lane + kWave] : 0.0f;
        ss = seg_sum<64>(lo);
        if (ngroups > kWave) ss += seg_sum<64>(hi);
    }
    const float inv = inv_rms(ss, p.inv_H, p.eps);

    __amdgpu_buffer_rsrc_t ro_ = rx, rsh = rx;
    if constexpr (MODE == kNormInPlace) ro_ = buf_rsrc((char*)p.x_out + ro, rb);
    if constexpr (MODE == kNormFp8)
        ro_ = buf_rsrc(p.y8 + (live ? row * (int64_t)p.H : 0), live ? (uint32_t)p.H : 0u);
    if constexpr (ADA) rsh = buf_rsrc((void*)p.shift, hb);
    float amax_acc = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int ch = k * stride + wir * kWave + lane;
        const uint32_t off = (uint32_t)ch * 16u;
        // (no residual: rr has range 0 and the store is dropped)
        if constexpr (MODE != kNormAmax) buf_st16_nt(rr, off, xv[k]);
        float s[V], wf[V], y[V];
        unpack<DT>(xv[k], s);
        unpack<DT>(wv[k], wf);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = (s[i] * inv) * (wf[i] + p.delta);
        if constexpr (ADA) {
            float sh[V];
            unpack<DT>(buf_ld16(rsh, off), sh);
#pragma unroll
            for (int i = 0; i < V; ++i) y[i] += sh[i];
        }
        if constexpr (MODE == kNormInPlace) {
            buf_st16_nt(ro_, off, pack<DT>(y));
        } else if constexpr (MODE == kNormFp8) {
            if constexpr (V == 8) {
                u32x2 c;
                c[0] = fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                             y[3] * p.inv_scale);
                c[1] = fp8x4(y[4] * p.inv_scale, y[5] * p.inv_scale, y[6] * p.inv_scale,
                             y[7] * p.inv_scale);
                buf_st8_nt(ro_, (uint32_t)ch * 8u, c);
            } else {
                buf_st4_nt(ro_, (uint32_t)ch * 4u,
                           fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                                 y[3] * p.inv_scale));
            }
        } else {
            const bool valid = live && ch < chunks;
#pragma unroll
            for (int i = 0; i < V; ++i) amax_acc = fmaxf(amax_acc, valid ? fabsf(y[i]) : 0.0f);
        }
    }
    if constexpr (MODE == kNormAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if (lane == 0 && live) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Half-chunk lanes: 16-bit rows of 65 to 256 chunks up to a few thousand
// waves.  With few rows most SIMDs are idle and a wave's arithmetic is its
// latency (each VALU instruction issues over 4 cycles), so each lane takes
// half a 16-byte chunk (8 bytes, 4 elements) and a row takes twice the
// waves: at most 8, two per SIMD of the row's CU (101 VALU instructions per
// wave against 168 for norm -> FP8).  Measured on MI355X, cold, bf16: norm -> FP8 H = 2048
// T = 1 / 128 2.09 / 2.57 -> 2.00 / 2.46 us; residual norm H = 1024 T = 1 /
// 128 1.97 / 2.39 -> 1.78 / 2.16 us.  At H = 2560 (ten waves on one CU) it
// measured no faster, so wider rows keep one chunk per lane.  The sums are
// the same bits as the other kernels': a chunk's FMA chain runs through its
// even lane (first four elements) and continues in the odd lane from the
// even lane's partial (one DPP move); with even lanes contributing zeros, a
// wave's 64-lane tree is the balanced tree over its 32 chunks, and the group
// tree's last level (a group's two 32-chunk halves) and the tree over groups
// are the tree over the waves' sums.  One row per block, one wave per 32
// chunks (p.wpr waves, at most 8).
template <int DT, int MODE>
__global__ __launch_bounds__(1024) void rmsnorm_half(NormParams p) {
    static_assert(DT != kF32, "16-bit dtypes");
    constexpr int EB = 2;
    __shared__ float hsum[8];
    asm volatile("" ::"s"(p.x), "s"(p.residual), "s"(p.w), "s"(p.H), "s"(p.eps), "s"(p.inv_H),
                 "s"(p.delta), "s"(p.wpr));
    if constexpr (MODE == kNormInPlace) asm volatile("" ::"s"(p.x_out));
    if constexpr (MODE == kNormFp8) asm volatile("" ::"s"(p.y8), "s"(p.inv_scale));
    if constexpr (MODE == kNormAmax) asm volatile("" ::"s"(p.amax));
    const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const int64_t row = blockIdx.x;
    const int chunks = p.H / 8;
    const bool has_res = p.residual != nullptr, has_w = p.w != nullptr;
    const uint32_t hb = (uint32_t)p.H * EB;
    const int64_t ro = row * (int64_t)hb;
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc((char*)p.x + ro, hb);
    const __amdgpu_buffer_rsrc_t rr =
        buf_rsrc(has_res ? (char*)p.residual + ro : (char*)p.x, has_res ? hb : 0u);
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc((void*)p.w, has_w ? hb : 0u);
    const uint32_t hc = (uint32_t)(wave * kWave + lane);     // half-chunk index
    const uint32_t off = hc * 8u;
    const u32x2 xv = buf_ld8_nt(rx, off);
    const u32x2 rv = buf_ld8_nt(rr, off);
    u32x2 wv = buf_ld8(rw, off);
    asm volatile("" ::: "memory");
    const uint32_t one = ones16<DT>()[0];
#pragma unroll
    for (int d = 0; d < 2; ++d) wv[d] = has_w ? wv[d] : one;

    // s = R(x + r), or x itself without a residual
    u32x2 sv;
    {
        u32x4 x4{xv[0], xv[1], 0u, 0u}, r4{rv[0], rv[1], 0u, 0u};
        float a[8], b[8];
        unpack<DT>(x4, a);
        unpack<DT>(r4, b);
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t sum = pack2<DT>(a[2 * d] + b[2 * d], a[2 * d + 1] + b[2 * d + 1]);
            sv[d] = has_res ? sum : xv[d];
        }
    }
    float s[8];
    unpack<DT>(u32x4{sv[0], sv[1], 0u, 0u}, s);
    // the chunk's chain: even lanes the first four elements, odd lanes the
    // last four from their partner's partial
    float pch = s[0] * s[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) pch = __builtin_fmaf(s[i], s[i], pch);
    float q = dpp<kDppQuadEven>(pch);
#pragma unroll
    for (int i = 0; i < 4; ++i) q = __builtin_fmaf(s[i], s[i], q);
    const float hs = seg_sum<64>((lane & 1) ? q : 0.0f);     // the wave's 32 chunks
    if (lane == 0) hsum[wave] = hs;
    __syncthreads();
    const float ss = seg_sum<64>(lane < p.wpr ? hsum[lane] : 0.0f);
    const float inv = inv_rms(ss, p.inv_H, p.eps);

    // (no residual: rr has range 0 and the store is dropped)
    if constexpr (MODE != kNormAmax) buf_st8_nt(rr, off, sv);
    float wf[8], y[4];
    unpack<DT>(u32x4{wv[0], wv[1], 0u, 0u}, wf);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (s[i] * inv) * (wf[i] + p.delta);
    if constexpr (MODE == kNormInPlace) {
        const u32x2 o{pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3])};
        buf_st8_nt(buf_rsrc((char*)p.x_out + ro, hb), off, o);
    } else if constexpr (MODE == kNormFp8) {
        buf_st4_nt(buf_rsrc(p.y8 + row * (int64_t)p.H, (uint32_t)p.H), hc * 4u,
                   fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                         y[3] * p.inv_scale));
    } else {
        const bool valid = (int)(hc >> 1) < chunks;
        float amax_acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) amax_acc = fmaxf(amax_acc, valid ? fabsf(y[i]) : 0.0f);
        amax_acc = seg_max<64>(amax_acc);
        if (lane == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Scalar kernel: any H and element-aligned pointers; one 256-thread block per
// row.  Pass 1: wave (g % 4) forms group g's chunk chains (Vec<DT> elements
// each, scalar loads) and its 64-lane tree; the group sums meet in LDS (up to
// kScalarGroups at a time, tree-summed; further blocks of groups are added in
// order).  Pass 2 recomputes s from the untouched x and r and writes, so each
// element is read before the same thread overwrites it.
constexpr int kScalarGroups = 1024;

template <int DT, int MODE, bool ADA>
__global__ __launch_bounds__(256) void rmsnorm_scalar(NormParams p) {
    constexpr int V = Vec<DT>::n;
    __shared__ float gsum[kScalarGroups];
    const int64_t row = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool has_res = p.residual != nullptr;
    const int64_t base = row * p.H;
    const int chunks = (p.H + V - 1) / V;
    const int ngroups = (chunks + kWave - 1) / kWave;
    float ss = 0.0f;
    for (int g0 = 0; g0 < ngroups; g0 += kScalarGroups) {
        const int gn = (ngroups - g0) < kScalarGroups ? (ngroups - g0) : kScalarGroups;
        for (int gi = wave; gi < gn; gi += 4) {
            const int c = (g0 + gi) * kWave + lane;
            float s[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int64_t e = (int64_t)c * V + i;
                float v = 0.0f;
                if (e < p.H) {
                    v = ld_elt<DT>(p.x, base + e);
                    if (ADA && p.gate) v = ld_elt<DT>(p.gate, e) * v;
                    if (has_res) v = round_trip<DT>(v + ld_elt<DT>(p.residual, base + e));
                }
                s[i] = v;
            }
            const float gsq = seg_sum<64>(chunk_sumsq<DT>(s));
            if (lane == 0) gsum[gi] = gsq;
        }
        __syncthreads();
        float blk = 0.0f;
        if (threadIdx.x == 0) blk = group_tree(gsum, gn);
        __syncthreads();
        if (threadIdx.x == 0) gsum[0] = blk;
        __syncthreads();
        ss = (g0 == 0) ? gsum[0] : ss + gsum[0];
        __syncthreads();
    }
    const float inv = inv_rms(ss, p.inv_H, p.eps);
    float amax_acc = 0.0f;
    for (int i = threadIdx.x; i < p.H; i += 256) {
        float s = ld_elt<DT>(p.x, base + i);
        if (ADA && p.gate) s = ld_elt<DT>(p.gate, i) * s;
        if (has_res) {
            s = round_trip<DT>(s + ld_elt<DT>(p.residual, base + i));
            if (MODE != kNormAmax) st_elt<DT>(p.residual, base + i, s);
        }
        float y = (s * inv) * ((p.w ? ld_elt<DT>(p.w, i) : 1.0f) + p.delta);
        if (ADA) y += ld_elt<DT>(p.shift, i);
        if constexpr (MODE == kNormInPlace) st_elt<DT>(p.x_out, base + i, y);
        else if constexpr (MODE == kNormFp8) p.y8[base + i] = fp8x1(y * p.inv_scale);
        else amax_acc = fmaxf(amax_acc, fabsf(y));
    }
    if constexpr (MODE == kNormAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if (lane == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Launch shape of the wide kernel: waves per row for a row of `chunks`
// 16-byte chunks.  One chunk per lane (as many waves as 64-chunk groups, the
// shortest per-wave latency) unless there are rows enough to fill the chip,
// then as few waves as kMaxNch chunks per lane allow (more would spill under
// the 1024-thread launch bound, which caps a wave at 128 VGPRs).

// Half-chunk lanes (rows of at most four 64-chunk groups) while the launch
// has at most this many waves (four per SIMD of 256 CUs).  Measured on
// MI355X, cold, bf16: up to this bound half-chunk lanes were faster at every
// width tried (norm -> FP8 H = 2048 T = 256 / 512 2.74 / 3.15 -> 2.61 / 3.07
// us; H = 1024 T = 1024 3.16 -> 2.96 us), above it slower (H = 2048 T = 1024
// 4.03 -> 4.13 us).
constexpr int64_t kHalfWaves = 4096;

int pick_wpr(int64_t T, int chunks) {
    // fewer waves per row once rows x 64-chunk groups reach this bound; the
    // bound is lower when a row's groups (one wave each) do not split evenly
    // over a CU's four SIMDs (H = 2560, 3584 in bf16; 1536, 2560 in fp32),
    // whose uneven blocks measured 4-20 % slower from about 5000 on
    constexpr int64_t wide_rows = 8192;
    constexpr int64_t wide_rows_uneven = 5000;
    const int per64 = (chunks + kWave - 1) / kWave;    // chunk groups
    const int min_wpr = (per64 + kMaxNch - 1) / kMaxNch;
    const int64_t bound = (per64 % 4) ? wide_rows_uneven : wide_rows;
    int wpr;
    if (T * per64 >= bound) wpr = min_wpr;
    else wpr = per64;
    if (wpr < min_wpr) wpr = min_wpr;
    if (wpr > 16) wpr = 16;
    if (wpr < 1) wpr = 1;
    return wpr;
}

template <int DT, int MODE, bool ADA, int NCH>
hipError_t launch_vec_n(const NormParams& p, hipStream_t s) {
    const int64_t blocks = (p.T + p.rpb - 1) / p.rpb;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_vec<DT, NCH, MODE, ADA>), dim3((uint32_t)blocks),
                       dim3(kWave * p.wpr * p.rpb), 0, s, p);
    return hipGetLastError();
}

template <int DT, int MODE, bool ADA, int G>
hipError_t launch_small(const NormParams& p, hipStream_t s) {
    constexpr int RPB = 4 * (kWave / G);                 // rows per 256-thread block
    const int64_t blocks = (p.T + RPB - 1) / RPB;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_small<DT, G, MODE, ADA>), dim3((uint32_t)blocks), dim3(256), 0,
                       s, p);
    return hipGetLastError();
}

template <int DT, int MODE, bool ADA>
hipError_t launch_mode(const NormArgs& a, hipStream_t s) {
    constexpr int V = Vec<DT>::n;
    NormParams p{};
    p.x = a.x; p.x_out = a.x_out; p.residual = a.residual; p.w = a.w; p.y8 = a.y8;
    p.amax = a.amax; p.inv_scale = a.inv_scale; p.T = a.T; p.H = a.H; p.eps = a.eps;
    p.inv_H = 1.0f / (float)a.H; p.delta = (float)a.weight_offset;
    p.gate = a.gate; p.shift = a.shift;

    const int chunks = a.H / V;
    bool vec = (a.H % V == 0) && chunks <= kMaxNch * kWave * 16 && aligned16(a.x) &&
               (a.w == nullptr || aligned16(a.w)) &&
               (a.residual == nullptr || aligned16(a.residual));
    if (ADA) vec = vec && (a.gate == nullptr || aligned16(a.gate)) && aligned16(a.shift);
    if (MODE == kNormInPlace) vec = vec && aligned16(a.x_out);
    if (MODE == kNormFp8)
        vec = vec && ((reinterpret_cast<uintptr_t>(a.y8) & (V == 8 ? 7u : 3u)) == 0);
    if (vec && chunks <= kWave) {
        if (chunks <= 4) return launch_small<DT, MODE, ADA, 4>(p, s);
        if (chunks <= 8) return launch_small<DT, MODE, ADA, 8>(p, s);
        if (chunks <= 16) return launch_small<DT, MODE, ADA, 16>(p, s);
        if (chunks <= 32) return launch_small<DT, MODE, ADA, 32>(p, s);
        return launch_small<DT, MODE, ADA, 64>(p, s);
    }
    if (vec && DT != kF32 && !ADA) {
        const int per64 = (chunks + kWave - 1) / kWave;
        if (per64 <= 4 && a.T * 2 * per64 <= kHalfWaves) {
            p.wpr = 2 * per64;
            hipLaunchKernelGGL((rmsnorm_half<DT == kF32 ? kBF16 : DT, MODE>), dim3((uint32_t)a.T),
                               dim3(kWave * p.wpr), 0, s, p);
            return hipGetLastError();
        }
    }
    if (vec) {
        p.wpr = pick_wpr(a.T, chunks);
        p.rpb = (p.wpr <= 4 && 4 % p.wpr == 0) ? 4 / p.wpr : 1;
        // several rows per block only for wpr 1, 2 or 4; one row: every
        // wave (at most 16) maps to row 0
        p.wsh = p.rpb > 1 ? (p.wpr == 1 ? 0 : (p.wpr == 2 ? 1 : 2)) : 5;
        const int nch = (chunks + kWave * p.wpr - 1) / (kWave * p.wpr);
        switch (nch) {
        case 1: return launch_vec_n<DT, MODE, ADA, 1>(p, s);
        case 2: return launch_vec_n<DT, MODE, ADA, 2>(p, s);
        case 3: return launch_vec_n<DT, MODE, ADA, 3>(p, s);
        case 4: return launch_vec_n<DT, MODE, ADA, 4>(p, s);
        case 5: return launch_vec_n<DT, MODE, ADA, 5>(p, s);
        default: return launch_vec_n<DT, MODE, ADA, 6>(p, s);
        }
    }
    if (a.T > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_scalar<DT, MODE, ADA>), dim3((uint32_t)a.T), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const NormArgs& a, hipStream_t s) {
    if (a.ada) {
        switch (a.mode) {
        case kNormInPlace: return launch_mode<DT, kNormInPlace, true>(a, s);
        case kNormFp8: return launch_mode<DT, kNormFp8, true>(a, s);
        default: return launch_mode<DT, kNormAmax, true>(a, s);
        }
    }
    switch (a.mode) {
    case kNormInPlace: return launch_mode<DT, kNormInPlace, false>(a, s);
    case kNormFp8: return launch_mode<DT, kNormFp8, false>(a, s);
    default: return launch_mode<DT, kNormAmax, false>(a, s);
    }
}

}  // namespace

hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t s) {
    switch (a.dtype) {
    case kF32: return launch_dt<kF32>(a, s);
    case kF16: return launch_dt<kF16>(a, s);
    default: return launch_dt<kBF16>(a, s);
    }
}

}  // namespace mbt
