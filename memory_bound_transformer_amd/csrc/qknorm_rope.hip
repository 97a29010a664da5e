// qknorm_rope.hip -- fused per-head QK-RMSNorm + rotary embedding prologue
// for gfx950.
//
// Operation ("thox-edge-ops v2", sections 5.1 and 5.4; ninfer PR #273,
// "Implementation"): every query head is RMS-normalised with w_q and every
// key head with w_k, the normalised value is rounded to the I/O dtype, and
// the first rot_dim channels of that rounded value are rotated by the cached
// angles of the token's position (rotate-half or interleaved pairs).  Tokens
// positioned beyond the cache get the norm only; their rotation is skipped.
//
// MI355X design (the pages' CUDA kernel -- one block per token, one warp per
// head, a block barrier between norm and rotation -- is prior art only):
//
//  * A head-row of D elements is a segment of G lanes of one wavefront; each
//    lane holds C 16-byte chunks (8 bf16 / fp16 or 4 fp32) strided by G, so
//    chunk group 0 (channels [0, G * Vec)) contains the whole rotated span
//    and only that chunk of each lane runs rotation code.  G * C * Vec = D.
//    Decode widths use C = 1 (most waves, least work per wave); prefill
//    widths use C = 4 where the rotated span allows (for D = 256, rot_dim 64
//    bf16: 8 lanes x 4 chunks per row, 8 rows per wave).
//  * A wave works on rows of ONE tensor (the q heads, then the k heads, each
//    flattened token-major), so a single set of norm weights sits in its
//    registers and the rows it streams are contiguous in memory.  Each lane
//    finds its row's token with a float reciprocal and one correction.
//  * The sum of squares reduces inside the G-lane segment with DPP (and the
//    gfx950 permlane swaps past 16 lanes); no LDS, no barrier.  The
//    normalised value stays in registers between the norm and the rotation,
//    so in-place calls are safe.
//  * Rotate-half pairs chunk j with chunk j + rot/2 / Vec; lanes 2j and
//    2j + 1 of a row hold that pair, so the partner arrives with one DPP quad
//    permute per dword.  Interleaved pairs are lane-local.
//  * q / k chunks are streamed with nontemporal loads and stores; weights,
//    positions and cos/sin rows use ordinary cached loads.
//  * Workgroups are renumbered so each of the 8 XCDs (dispatched round-robin)
//    gets a contiguous range of rows.
//
// A scalar kernel (one wave per head-row, LDS-staged rotation) covers every
// shape and alignment the vector kernel does not; both give identical
// results up to the reduction order of the fp32 sum of squares.

#include <stdlib.h>

#include "mbt_device.hpp"
#include "mbt_launch.hpp"

namespace mbt {
namespace {

struct QkParams {
    const void* q_in;
    const void* k_in;
    void* q_out;
    void* k_out;
    const void* w_q;
    const void* w_k;
    const float* cos_sin;
    const int64_t* pos;
    int64_t max_pos;
    int64_t T;
    int32_t Q, K, D, rot;
    float eps, inv_D, delta;
    int32_t layout;           // 0 rotate-half, 1 interleaved
    float inv_Q, inv_K;       // vector kernel: 1/Q, 1/K for the token index
    uint32_t q_waves;         // vector kernel: waves over the T*Q query rows
    uint32_t total_waves;     // vector kernel: q_waves + waves over key rows
    uint32_t n_blocks;
};

// Vector kernel.  DT: dtype; G: lanes per head-row; C: chunks per lane
// (G * C * Vec<DT> = D); LAYOUT: rotary pairing.  Requires 16-byte aligned
// q / k / w tensors, every rotated chunk inside chunk group 0, rows of each
// tensor below 2^24, and for rotate-half rot/2 a multiple of Vec<DT> with a
// 16-byte aligned cos/sin cache (interleaved reads its run element-wise).
template <int DT, int G, int C, int LAYOUT>
__global__ __launch_bounds__(256) void qknorm_rope_vec(QkParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int RPW = kWave / G;     // rows per wave
    constexpr int EB = EltBytes<DT>::n;
    // C >= 2: the fp32 (w + delta) vectors live in LDS, not in 2 * C * V
    // registers per lane, which keeps these kernels at 8 waves per SIMD.
    __shared__ float wsh[C >= 2 ? 2 : 1][C >= 2 ? 512 : 1];

    const uint32_t lb = xcd_remap(blockIdx.x, p.n_blocks);
    const uint32_t wv = (uint32_t)uniform((int)(lb * 4u + (threadIdx.x >> 6)));
    const bool wave_live = wv < p.total_waves;
    const bool is_q = wv < p.q_waves;                       // wave-uniform tensor
    const int heads = is_q ? p.Q : p.K;
    const float inv_heads = is_q ? p.inv_Q : p.inv_K;
    const int64_t nrows = wave_live ? p.T * heads : 0;
    const int64_t row0 = (int64_t)(is_q ? wv : wv - p.q_waves) * RPW;
    const char* src = (const char*)(is_q ? p.q_in : p.k_in);
    char* dst = (char*)(is_q ? p.q_out : p.k_out);
    const char* wp = (const char*)(is_q ? p.w_q : p.w_k);

    const int lane = threadIdx.x & 63;
    const int j = lane % G;                                 // lane within the row
    const int64_t row = row0 + lane / G;
    const bool live = row < nrows;
    const int half = p.rot >> 1;

    // chunk of group 0 held by this lane, and its rotation role
    int c0 = j;
    bool is_a = false, is_b = false;
    if constexpr (LAYOUT == 0) {
        const int hv = half / V;
        if (j < 2 * hv) {
            is_a = (j & 1) == 0;
            is_b = !is_a;
            c0 = is_a ? (j >> 1) : hv + (j >> 1);
        }
    }
    auto chunk = [&](int k) { return k == 0 ? c0 : k * G + j; };

    // ---- issue every independent load before any arithmetic ----
    const char* rsrc = src + row * (int64_t)p.D * EB;
    u32x4 x[C];
#pragma unroll
    for (int k = 0; k < C; ++k)
        x[k] = live ? ld16_nt(rsrc + chunk(k) * 16) : u32x4{0u, 0u, 0u, 0u};
    // token of the row: float reciprocal, then one correction each way
    const uint32_t r32 = live ? (uint32_t)row : 0u;
    int32_t t = (int32_t)((float)r32 * inv_heads);
    const int32_t rem = (int32_t)r32 - t * heads;
    t += (rem >= heads) ? 1 : 0;
    t -= (rem < 0) ? 1 : 0;
    const int64_t ppos = live ? p.pos[t] : -1;
    float wreg[C >= 2 ? 1 : V];
    if constexpr (C >= 2) {
        for (int i = threadIdx.x; i < p.D; i += 256) {
            wsh[0][i] = (p.Q > 0) ? ld_elt<DT>(p.w_q, i) + p.delta : 0.0f;
            wsh[1][i] = (p.K > 0) ? ld_elt<DT>(p.w_k, i) + p.delta : 0.0f;
        }
        __syncthreads();                                   // x loads already in flight
    } else {
        unpack<DT>(wave_live ? ld16(wp + c0 * 16) : u32x4{0u, 0u, 0u, 0u}, wreg);
#pragma unroll
        for (int i = 0; i < V; ++i) wreg[i] += p.delta;
    }
    if (!wave_live) return;
    const bool rotate = (ppos >= 0) && (ppos < p.max_pos) && (p.rot > 0);
    float cs_c[V], cs_s[V];
    bool lane_rot = false;
    if constexpr (LAYOUT == 0) {
        lane_rot = rotate && (is_a || is_b);
        if (lane_rot) {
            const int j0 = (j >> 1) * V;                    // first pair index
            const float* crow = p.cos_sin + ppos * (int64_t)p.rot;
#pragma unroll
            for (int i = 0; i < V; i += 4) {
                const u32x4 cv = ld16(crow + j0 + i);
                const u32x4 sv = ld16(crow + half + j0 + i);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    cs_c[i + k] = __uint_as_float(cv[k]);
                    // sign folded in: o = own * c + partner * s'
                    cs_s[i + k] = is_a ? -__uint_as_float(sv[k]) : __uint_as_float(sv[k]);
                }
            }
        }
    } else {
        const int j0 = c0 * (V / 2);                        // first pair index
        lane_rot = rotate && (j0 < half);
        if (lane_rot) {
            const float* crow = p.cos_sin + ppos * (int64_t)p.rot;
            // V/2 pairs per lane; a run may cross rot/2, so read against the
            // bound (pairs past it keep c = 1, s = 0: exactly unrotated).
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                const bool ok = (j0 + i) < half;
                cs_c[i] = ok ? crow[j0 + i] : 1.0f;
                cs_s[i] = ok ? crow[half + j0 + i] : 0.0f;
            }
        }
    }

    // ---- norm, round, rotate (group 0 only), store ----
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
        float f[V];
        unpack<DT>(x[k], f);
#pragma unroll
        for (int i = 0; i < V; ++i) ss += f[i] * f[i];
    }
    ss = seg_sum<G>(ss);
    const float inv = rsqrt_hw(ss * p.inv_D + p.eps);
    char* rdst = dst + row * (int64_t)p.D * EB;
    const float* wrow = wsh[(C >= 2 && !is_q) ? 1 : 0];
#pragma unroll
    for (int k = 0; k < C; ++k) {
        float f[V], n[V];
        unpack<DT>(x[k], f);                                // decoded again: fewer live VGPRs
        if constexpr (C >= 2) {
            const float* wk = wrow + chunk(k) * V;
#pragma unroll
            for (int i = 0; i < V; ++i) n[i] = (f[i] * inv) * wk[i];
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) n[i] = (f[i] * inv) * wreg[i];
        }
        u32x4 out = pack<DT>(n);                            // R(n): the rounded value
        if (k == 0) {
            if constexpr (LAYOUT == 0) {
                u32x4 pb;                                   // partner: neighbouring lane
#pragma unroll
                for (int d = 0; d < 4; ++d) pb[d] = dpp_u<kDppQuadXor1>(out[d]);
                if (lane_rot) {
                    float a[V], b[V], o[V];
                    unpack<DT>(out, a);
                    unpack<DT>(pb, b);
#pragma unroll
                    for (int i = 0; i < V; ++i) o[i] = a[i] * cs_c[i] + b[i] * cs_s[i];
                    out = pack<DT>(o);
                }
            } else {
                if (lane_rot) {
                    float a[V], o[V];
                    unpack<DT>(out, a);
#pragma unroll
                    for (int i = 0; i < V / 2; ++i) {
                        o[2 * i] = a[2 * i] * cs_c[i] - a[2 * i + 1] * cs_s[i];
                        o[2 * i + 1] = a[2 * i + 1] * cs_c[i] + a[2 * i] * cs_s[i];
                    }
                    out = pack<DT>(o);
                }
            }
        }
        if (live) st16_nt(rdst + chunk(k) * 16, out);
    }
}

// Scalar kernel: any D <= 512, any even rot, element-aligned pointers.  One
// wave per head-row (4 rows per 256-thread block); lane i owns elements
// i, i + 64, ...; the rounded normalised row is staged in LDS so each lane
// can read its rotation partner.
template <int DT>
__global__ __launch_bounds__(256) void qknorm_rope_scalar(QkParams p) {
    __shared__ float stage[4][512];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + w;
    const int QK = p.Q + p.K;
    const int64_t rows = p.T * QK;
    const bool live = row < rows;
    const int64_t t = live ? row / QK : 0;
    const int h = live ? (int)(row % QK) : 0;
    const bool is_q = h < p.Q;
    const void* src = is_q ? p.q_in : p.k_in;
    void* dst = is_q ? p.q_out : p.k_out;
    const void* wp = is_q ? p.w_q : p.w_k;
    const int64_t base = is_q ? (t * p.Q + h) * (int64_t)p.D
                              : (t * p.K + (h - p.Q)) * (int64_t)p.D;
    constexpr int MAXE = 512 / kWave;
    float f[MAXE];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < MAXE; ++k) {
        const int i = lane + k * kWave;
        f[k] = (live && i < p.D) ? ld_elt<DT>(src, base + i) : 0.0f;
        ss += f[k] * f[k];
    }
    ss = seg_sum<64>(ss);
    const float inv = rsqrt_hw(ss * p.inv_D + p.eps);
#pragma unroll
    for (int k = 0; k < MAXE; ++k) {
        const int i = lane + k * kWave;
        if (live && i < p.D)
            stage[w][i] = round_trip<DT>((f[k] * inv) * (ld_elt<DT>(wp, i) + p.delta));
    }
    __syncthreads();
    if (!live) return;
    const int64_t ppos = p.pos[t];
    const bool rotate = (ppos >= 0) && (ppos < p.max_pos) && (p.rot > 0);
    const int half = p.rot >> 1;
    const float* cs = p.cos_sin + (rotate ? ppos * (int64_t)p.rot : 0);
#pragma unroll
    for (int k = 0; k < MAXE; ++k) {
        const int i = lane + k * kWave;
        if (i >= p.D) continue;
        float o = stage[w][i];
        if (rotate && i < p.rot) {
            int j, a, b;
            if (p.layout == 0) {                     // rotate-half
                j = (i < half) ? i : i - half;
                a = j;
                b = j + half;
            } else {                                 // interleaved
                j = i >> 1;
                a = 2 * j;
                b = 2 * j + 1;
            }
            const float c = cs[j], s = cs[half + j];
            o = (i == a) ? (stage[w][a] * c - stage[w][b] * s)
                         : (stage[w][b] * c + stage[w][a] * s);
        }
        st_elt<DT>(dst, base + i, o);
    }
}

// Launch-shape tunable, read once from the environment (sweeps only; the
// default is the measured best on MI355X).
int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}
int tun_strided_rows() {
    static const int v = env_int("MBT_QK_STRIDED_ROWS", 4096);
    return v;
}
int tun_c_max() {
    static const int v = env_int("MBT_QK_C_MAX", 4);
    return v;
}

template <int DT, int G, int C, int LAYOUT>
hipError_t launch_vec(const QkParams& p0, hipStream_t s) {
    QkParams p = p0;
    constexpr int RPW = kWave / G;
    const int64_t qw = (p.T * p.Q + RPW - 1) / RPW;
    const int64_t kw = (p.T * p.K + RPW - 1) / RPW;
    p.q_waves = (uint32_t)qw;
    p.total_waves = (uint32_t)(qw + kw);
    p.n_blocks = (p.total_waves + 3u) / 4u;
    hipLaunchKernelGGL((qknorm_rope_vec<DT, G, C, LAYOUT>), dim3(p.n_blocks), dim3(256), 0, s,
                       p);
    return hipGetLastError();
}

// (G, C) with G * C = L lanes-of-chunks per row; G a power of two >= 4.
template <int DT, int LAYOUT>
hipError_t launch_gc(const QkParams& p, int L, int C, hipStream_t s) {
#define MBT_QK_CASE(LL, CC)                                              \
    if (L == LL && C == CC) return launch_vec<DT, LL / CC, CC, LAYOUT>(p, s);
    MBT_QK_CASE(4, 1)
    MBT_QK_CASE(8, 1) MBT_QK_CASE(8, 2)
    MBT_QK_CASE(16, 1) MBT_QK_CASE(16, 2) MBT_QK_CASE(16, 4)
    MBT_QK_CASE(32, 1) MBT_QK_CASE(32, 2) MBT_QK_CASE(32, 4)
    MBT_QK_CASE(64, 1) MBT_QK_CASE(64, 2) MBT_QK_CASE(64, 4)
#undef MBT_QK_CASE
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const QkArgs& a, hipStream_t s) {
    constexpr int V = Vec<DT>::n;
    QkParams p{};
    p.q_in = a.q_in; p.k_in = a.k_in; p.q_out = a.q_out; p.k_out = a.k_out;
    p.w_q = a.w_q; p.w_k = a.w_k; p.cos_sin = a.cos_sin; p.pos = a.pos;
    p.max_pos = a.max_pos; p.T = a.T; p.Q = a.Q; p.K = a.K; p.D = a.head_dim;
    p.rot = a.rot_dim; p.eps = a.eps; p.inv_D = 1.0f / (float)a.head_dim;
    p.delta = (float)a.weight_offset;
    p.layout = a.layout;

    // Vector path conditions.
    const int L = a.head_dim / V;
    bool vec = (a.head_dim % V == 0) && (L == 4 || L == 8 || L == 16 || L == 32 || L == 64);
    vec = vec && aligned16(a.q_in) && aligned16(a.k_in) && aligned16(a.q_out) &&
          aligned16(a.k_out) && aligned16(a.w_q) && aligned16(a.w_k);
    if (a.rot_dim > 0 && a.max_pos > 0) {
        if (a.layout == 0)
            vec = vec && ((a.rot_dim / 2) % V == 0) && aligned16(a.cos_sin) &&
                  (a.rot_dim % 4 == 0);
        else
            vec = vec && aligned16(a.cos_sin);
    }
    const int QK = a.Q + a.K;
    const int64_t rows = a.T * (int64_t)QK;
    // rows of each tensor below 2^24: the token index uses a float reciprocal
    vec = vec && a.T * (int64_t)(a.Q > a.K ? a.Q : a.K) < (int64_t(1) << 24);
    if (vec) {
        // Chunks per lane: 1 at decode widths; at prefill widths up to 4,
        // as long as the rotated span stays inside chunk group 0 (G lanes).
        const int half = a.rot_dim / 2;
        const int rc = (a.rot_dim == 0) ? 0
                       : (a.layout == 0 ? 2 * (half / V) : (a.rot_dim + V - 1) / V);
        int C = 1;
        if (rows >= tun_strided_rows()) {
            for (int cand : {4, 2}) {
                const int G = L / cand;
                if (cand <= tun_c_max() && G >= 4 && G >= rc) { C = cand; break; }
            }
        }
        p.inv_Q = a.Q > 0 ? 1.0f / (float)a.Q : 0.0f;
        p.inv_K = a.K > 0 ? 1.0f / (float)a.K : 0.0f;
        return (a.layout == 0) ? launch_gc<DT, 0>(p, L, C, s) : launch_gc<DT, 1>(p, L, C, s);
    }
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qknorm_rope_scalar<DT>), dim3((uint32_t)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope(const QkArgs& a, hipStream_t s) {
    switch (a.dtype) {
    case kF32: return launch_dt<kF32>(a, s);
    case kF16: return launch_dt<kF16>(a, s);
    default: return launch_dt<kBF16>(a, s);
    }
}

}  // namespace mbt
