// rmsnorm.hip -- fused residual-add RMSNorm for gfx950, with an in-place
// dtype output, a static-scale OCP e4m3fn output, or a calibration amax.
//
// Operation ("thox-edge-ops v2", section 5.1: one kernel stores the sum back
// into the residual stream and normalises that rounded sum; section 3, R1:
// the stored sum equals an eager elementwise add bit for bit):
//   s = R(x + r);  r <- s;  x <- R((s * inv) * (w + delta)),
//   inv = 1 / sqrt(mean(s^2) + eps).
// FP8 epilogue (FlashRT optimization details, fused kernel table and static
// FP8 calibration): y = E4M3FN(((s * inv) * (w + delta)) * inv_scale) with x
// left unchanged; the calibration pass instead folds max |(s*inv)*(w+delta)|
// into a device scalar and writes nothing else.
//
// MI355X design: the row stays in registers from load to store (the single
// read pass the FlashRT notes credit for their norm speed-up), so HBM sees exactly
// one read of x, r, w and one write of r and the output.  A row of H
// elements is spread over WPR waves of NCH 16-byte chunks per lane; the
// fp32 sum of squares reduces inside each wave with DPP and, only when
// WPR > 1, across waves through LDS with one barrier.  With WPR == 1 a
// 256-thread block carries four independent rows and no barrier at all.
// Odd widths and unaligned pointers take a two-pass scalar kernel with the
// same arithmetic.

#include <stdlib.h>

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
    int32_t wpr;   // waves per row
    int32_t rpb;   // rows per block
};

template <int DT, int MODE>
__device__ __forceinline__ void emit(const NormParams& p, int64_t row, int64_t e0,
                                     const float* y, float& amax_acc) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    if constexpr (MODE == kNormInPlace) {
        st16_nt((char*)p.x_out + (row * p.H + e0) * EB, pack<DT>(y));
    } else if constexpr (MODE == kNormFp8) {
        uint8_t* dst = p.y8 + row * p.H + e0;
        if constexpr (V == 8) {
            u32x2 c;
            c[0] = fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                         y[3] * p.inv_scale);
            c[1] = fp8x4(y[4] * p.inv_scale, y[5] * p.inv_scale, y[6] * p.inv_scale,
                         y[7] * p.inv_scale);
            st8_nt(dst, c);
        } else {
            st4_nt(dst, fp8x4(y[0] * p.inv_scale, y[1] * p.inv_scale, y[2] * p.inv_scale,
                              y[3] * p.inv_scale));
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) amax_acc = fmaxf(amax_acc, fabsf(y[i]));
    }
}

// Vector kernel: H a multiple of Vec<DT>, 16-byte aligned x / residual / w /
// x_out, and (FP8) y8 aligned to its store width.
template <int DT, int NCH, int MODE>
__global__ __launch_bounds__(1024) void rmsnorm_vec(NormParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    __shared__ float part[16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wpr = p.wpr;
    const int rib = wave / wpr, wir = wave % wpr;
    const int64_t row = (int64_t)blockIdx.x * p.rpb + rib;
    const bool live = row < p.T;
    const int chunks = p.H / V;
    const int stride = kWave * wpr;
    const bool has_res = p.residual != nullptr;

    // Every load of the row (x, residual, weight) is issued before any math.
    u32x4 xv[NCH], rv[NCH], wv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int ch = k * stride + wir * kWave + lane;
        xv[k] = u32x4{0u, 0u, 0u, 0u};
        rv[k] = u32x4{0u, 0u, 0u, 0u};
        wv[k] = u32x4{0u, 0u, 0u, 0u};
        if (live && ch < chunks) {
            const int64_t off = (row * p.H + (int64_t)ch * V) * EB;
            xv[k] = ld16_nt((const char*)p.x + off);
            if (has_res) rv[k] = ld16_nt((const char*)p.residual + off);
            wv[k] = ld16((const char*)p.w + (int64_t)ch * V * EB);
        }
    }
    // s = R(x + r): fp32 add of the decoded operands, one rounding.
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        if (has_res) {
            float a[V], b[V];
            unpack<DT>(xv[k], a);
            unpack<DT>(rv[k], b);
#pragma unroll
            for (int i = 0; i < V; ++i) a[i] += b[i];
            xv[k] = pack<DT>(a);          // xv now holds the rounded sum s
        }
        float s[V];
        unpack<DT>(xv[k], s);
#pragma unroll
        for (int i = 0; i < V; ++i) ss += s[i] * s[i];
    }
    ss = seg_sum<64>(ss);
    if (wpr > 1) {
        if (lane == 0) part[wave] = ss;
        __syncthreads();
        ss = 0.0f;
        for (int i = 0; i < wpr; ++i) ss += part[rib * wpr + i];
    }
    const float inv = rsqrt_hw(ss * p.inv_H + p.eps);
    float amax_acc = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int ch = k * stride + wir * kWave + lane;
        if (!(live && ch < chunks)) continue;
        const int64_t e0 = (int64_t)ch * V;
        if (has_res && MODE != kNormAmax)
            st16_nt((char*)p.residual + (row * p.H + e0) * EB, xv[k]);
        float s[V], wf[V], y[V];
        unpack<DT>(xv[k], s);
        unpack<DT>(wv[k], wf);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = (s[i] * inv) * (wf[i] + p.delta);
        emit<DT, MODE>(p, row, e0, y, amax_acc);
    }
    if constexpr (MODE == kNormAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if (lane == 0 && live) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Scalar kernel: any H and element-aligned pointers.  One 256-thread block
// per row; the first pass forms s and its sum of squares, the second pass
// recomputes s from the untouched x and r and writes everything, so each
// element is read before it is overwritten by the same thread.
template <int DT, int MODE>
__global__ __launch_bounds__(256) void rmsnorm_scalar(NormParams p) {
    __shared__ float part[4];
    const int64_t row = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool has_res = p.residual != nullptr;
    const int64_t base = row * p.H;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < p.H; i += 256) {
        float s = ld_elt<DT>(p.x, base + i);
        if (has_res) s = round_trip<DT>(s + ld_elt<DT>(p.residual, base + i));
        ss += s * s;
    }
    ss = seg_sum<64>(ss);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    ss = part[0] + part[1] + part[2] + part[3];
    const float inv = rsqrt_hw(ss * p.inv_H + p.eps);
    float amax_acc = 0.0f;
    for (int i = threadIdx.x; i < p.H; i += 256) {
        float s = ld_elt<DT>(p.x, base + i);
        if (has_res) {
            s = round_trip<DT>(s + ld_elt<DT>(p.residual, base + i));
            if (MODE != kNormAmax) st_elt<DT>(p.residual, base + i, s);
        }
        const float y = (s * inv) * (ld_elt<DT>(p.w, i) + p.delta);
        if constexpr (MODE == kNormInPlace) st_elt<DT>(p.x_out, base + i, y);
        else if constexpr (MODE == kNormFp8) p.y8[base + i] = fp8x1(y * p.inv_scale);
        else amax_acc = fmaxf(amax_acc, fabsf(y));
    }
    if constexpr (MODE == kNormAmax) {
        amax_acc = seg_max<64>(amax_acc);
        if (lane == 0) atomic_max_nonneg(p.amax, amax_acc);
    }
}

// Launch shape: waves per row for a row of `chunks` 16-byte chunks.
// Decode widths (few rows) spread each row over as many waves as it has
// 64-chunk groups, one chunk per lane (the shortest per-wave latency);
// prefill widths keep a row in as few waves as kMaxNch chunks per lane
// allow (more chunks per lane would spill under the 1024-thread launch
// bound, which caps a wave at 128 VGPRs).
constexpr int kMaxNch = 6;

int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}

int pick_wpr(int64_t T, int chunks) {
    static const int forced = env_int("MBT_NORM_WPR", 0);
    static const int wide_rows = env_int("MBT_NORM_WIDE_CHUNKS", 32768);
    const int per64 = (chunks + kWave - 1) / kWave;    // chunks per lane at WPR 1
    const int min_wpr = (per64 + kMaxNch - 1) / kMaxNch;
    int wpr;
    if (forced > 0) wpr = forced;
    else if (T * per64 >= wide_rows) wpr = min_wpr;    // enough rows to fill the chip
    else wpr = per64;                                   // one chunk per lane
    if (wpr < min_wpr) wpr = min_wpr;
    if (wpr > 16) wpr = 16;
    if (wpr < 1) wpr = 1;
    return wpr;
}

template <int DT, int MODE, int NCH>
hipError_t launch_vec_n(const NormParams& p, hipStream_t s) {
    const int64_t blocks = (p.T + p.rpb - 1) / p.rpb;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_vec<DT, NCH, MODE>), dim3((uint32_t)blocks),
                       dim3(kWave * p.wpr * p.rpb), 0, s, p);
    return hipGetLastError();
}

template <int DT, int MODE>
hipError_t launch_mode(const NormArgs& a, hipStream_t s) {
    constexpr int V = Vec<DT>::n;
    NormParams p{};
    p.x = a.x; p.x_out = a.x_out; p.residual = a.residual; p.w = a.w; p.y8 = a.y8;
    p.amax = a.amax; p.inv_scale = a.inv_scale; p.T = a.T; p.H = a.H; p.eps = a.eps;
    p.inv_H = 1.0f / (float)a.H; p.delta = (float)a.weight_offset;

    const int chunks = a.H / V;
    bool vec = (a.H % V == 0) && chunks <= kMaxNch * kWave * 16 && aligned16(a.x) &&
               aligned16(a.w) &&
               (a.residual == nullptr || aligned16(a.residual));
    if (MODE == kNormInPlace) vec = vec && aligned16(a.x_out);
    if (MODE == kNormFp8)
        vec = vec && ((reinterpret_cast<uintptr_t>(a.y8) & (V == 8 ? 7u : 3u)) == 0);
    if (vec) {
        p.wpr = pick_wpr(a.T, chunks);
        p.rpb = (p.wpr <= 4 && 4 % p.wpr == 0) ? 4 / p.wpr : 1;
        const int nch = (chunks + kWave * p.wpr - 1) / (kWave * p.wpr);
        switch (nch) {
        case 1: return launch_vec_n<DT, MODE, 1>(p, s);
        case 2: return launch_vec_n<DT, MODE, 2>(p, s);
        case 3: return launch_vec_n<DT, MODE, 3>(p, s);
        case 4: return launch_vec_n<DT, MODE, 4>(p, s);
        case 5: return launch_vec_n<DT, MODE, 5>(p, s);
        default: return launch_vec_n<DT, MODE, 6>(p, s);
        }
    }
    if (a.T > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_scalar<DT, MODE>), dim3((uint32_t)a.T), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const NormArgs& a, hipStream_t s) {
    switch (a.mode) {
    case kNormInPlace: return launch_mode<DT, kNormInPlace>(a, s);
    case kNormFp8: return launch_mode<DT, kNormFp8>(a, s);
    default: return launch_mode<DT, kNormAmax>(a, s);
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
