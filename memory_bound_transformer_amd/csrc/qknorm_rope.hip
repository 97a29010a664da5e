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
//  * A head-row of D elements is a segment of L = D / (16 B / elt) lanes of
//    one wavefront, each lane holding one 16-byte chunk (8 bf16 / fp16 or 4
//    fp32).  D = 256 bf16 is 32 lanes, so a wave64 covers RPW = 64 / L rows
//    per step; a wave runs U steps over consecutive heads of ONE token, so
//    the position, the cos/sin row and both weight chunks are loaded once
//    per wave and every x load of the U steps is issued before any math.
//  * The sum of squares reduces inside the segment with DPP (no LDS, no
//    barrier); the rotate-half partner chunk (rot_dim/2 channels away) sits
//    in another lane of the same segment and is fetched with one lane
//    shuffle per dword; interleaved pairs are lane-local.
//  * There is no barrier anywhere: the normalised value stays in registers
//    between the norm and the rotation, so in-place calls are safe.
//  * Workgroups are renumbered so each of the 8 XCDs (dispatched round-robin)
//    gets a contiguous range of tokens: a token's cos/sin row and position
//    are then fetched into one XCD's L2 instead of several.
//
// A scalar kernel (one wave per head-row, LDS-staged rotation) covers every
// shape and alignment the vector kernel does not; both give identical
// results up to the reduction order of the fp32 sum of squares.

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
    int32_t units_per_token;  // vector kernel: waves per token
    int32_t heads_per_unit;   // vector kernel: RPW * U
    uint32_t total_units;     // T * units_per_token
    uint32_t n_blocks;
};

// Vector kernel.  DT: dtype; L: lanes per head-row; LAYOUT: rotary pairing;
// U: steps per wave.  Requires 16-byte aligned tensors, D = L * Vec<DT>,
// and for rotate-half rot/2 a multiple of Vec<DT>; for interleaved, rot a
// multiple of 4 (so each lane's cos/sin run is 8-byte aligned).
template <int DT, int L, int LAYOUT, int U>
__global__ __launch_bounds__(256) void qknorm_rope_vec(QkParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int RPW = kWave / L;
    constexpr int EB = EltBytes<DT>::n;

    // XCD-aware renumbering: hardware block b runs on XCD b % 8, so XCD x
    // receives hardware blocks x, x + 8, ...; give it the logical blocks
    // [base(x), base(x) + count(x)) instead (a bijection on [0, nb)).
    const uint32_t lb = xcd_remap(blockIdx.x, p.n_blocks);
    const uint32_t unit = (uint32_t)uniform((int)(lb * 4u + (threadIdx.x >> 6)));
    if (unit >= p.total_units) return;

    const uint32_t upt = (uint32_t)p.units_per_token;
    const int64_t t = (int64_t)(unit / upt);
    const int head0 = (int)(unit % upt) * p.heads_per_unit;
    const int lane = threadIdx.x & 63;
    const int seg = lane / L;          // row within a step
    const int c = lane % L;            // chunk within the row
    const int QK = p.Q + p.K;

    // ---- issue every load before any arithmetic ----
    const int64_t ppos = p.pos[t];
    u32x4 x[U];
    int head[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        head[u] = head0 + u * RPW + seg;
        x[u] = u32x4{0u, 0u, 0u, 0u};
        if (head[u] < QK) {
            const char* src = (head[u] < p.Q)
                ? (const char*)p.q_in + ((t * p.Q + head[u]) * (int64_t)p.D) * EB
                : (const char*)p.k_in + ((t * p.K + (head[u] - p.Q)) * (int64_t)p.D) * EB;
            x[u] = ld16(src + c * 16);
        }
    }
    float wq[V], wk[V];
    {
        u32x4 a = (p.Q > 0) ? ld16((const char*)p.w_q + c * 16) : u32x4{0u, 0u, 0u, 0u};
        u32x4 bb = (p.K > 0) ? ld16((const char*)p.w_k + c * 16) : u32x4{0u, 0u, 0u, 0u};
        unpack<DT>(a, wq);
        unpack<DT>(bb, wk);
#pragma unroll
        for (int i = 0; i < V; ++i) { wq[i] += p.delta; wk[i] += p.delta; }
    }
    const bool rotate = (ppos >= 0) && (ppos < p.max_pos) && (p.rot > 0);
    const int half = p.rot >> 1;
    // This lane's rotation role and its cos/sin run.
    float cs_c[V], cs_s[V];
    bool lane_rot = false;
    int partner = lane;
    if constexpr (LAYOUT == 0) {
        const int hv = half / V;                     // partner distance in lanes
        const bool is_a = c < hv, is_b = (c >= hv) && (c < 2 * hv);
        lane_rot = rotate && (is_a || is_b);
        partner = is_a ? lane + hv : (is_b ? lane - hv : lane);
        if (lane_rot) {
            const int j0 = (is_a ? c : c - hv) * V;  // first pair index
            const float* row = p.cos_sin + ppos * (int64_t)p.rot;
#pragma unroll
            for (int i = 0; i < V; i += 4) {
                u32x4 cv = ld16(row + j0 + i);
                u32x4 sv = ld16(row + half + j0 + i);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    cs_c[i + k] = __uint_as_float(cv[k]);
                    cs_s[i + k] = __uint_as_float(sv[k]);
                }
            }
        }
    } else {
        const int j0 = c * (V / 2);                  // first pair index
        lane_rot = rotate && (j0 < half);
        if (lane_rot) {
            const float* row = p.cos_sin + ppos * (int64_t)p.rot;
            // V/2 pairs: 2 (fp32) or 4 (16-bit) cos and sin values; the run
            // may cross rot/2 only when rot/2 is not a multiple of V/2, so
            // read element-wise against the bound.
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                const bool ok = (j0 + i) < half;
                cs_c[i] = ok ? row[j0 + i] : 1.0f;
                cs_s[i] = ok ? row[half + j0 + i] : 0.0f;
            }
        }
    }

    // ---- per step: norm, round, rotate, store ----
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float f[V];
        unpack<DT>(x[u], f);
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i) ss += f[i] * f[i];
        ss = seg_sum<L>(ss);
        const float inv = rsqrt_hw(ss * p.inv_D + p.eps);
        const bool is_q = head[u] < p.Q;
        float n[V];
#pragma unroll
        for (int i = 0; i < V; ++i) n[i] = (f[i] * inv) * (is_q ? wq[i] : wk[i]);
        u32x4 nb16 = pack<DT>(n);                    // R(n): the rounded value
        u32x4 out = nb16;
        if constexpr (LAYOUT == 0) {
            // partner chunk of the same row (other half of the rotated span)
            u32x4 pb;
#pragma unroll
            for (int k = 0; k < 4; ++k) pb[k] = (uint32_t)__shfl((int)nb16[k], partner, 64);
            if (lane_rot) {
                float a[V], o[V], bq[V];
                unpack<DT>(nb16, a);
                unpack<DT>(pb, bq);
                const bool is_a = partner > lane;
#pragma unroll
                for (int i = 0; i < V; ++i)
                    o[i] = is_a ? (a[i] * cs_c[i] - bq[i] * cs_s[i])
                                : (a[i] * cs_c[i] + bq[i] * cs_s[i]);
                out = pack<DT>(o);
            }
        } else {
            if (lane_rot) {
                float a[V], o[V];
                unpack<DT>(nb16, a);
#pragma unroll
                for (int i = 0; i < V / 2; ++i) {
                    o[2 * i] = a[2 * i] * cs_c[i] - a[2 * i + 1] * cs_s[i];
                    o[2 * i + 1] = a[2 * i + 1] * cs_c[i] + a[2 * i] * cs_s[i];
                }
                out = pack<DT>(o);
            }
        }
        if (head[u] < QK) {
            char* dst = is_q
                ? (char*)p.q_out + ((t * p.Q + head[u]) * (int64_t)p.D) * EB
                : (char*)p.k_out + ((t * p.K + (head[u] - p.Q)) * (int64_t)p.D) * EB;
            st16(dst + c * 16, out);
        }
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

template <int DT, int L, int LAYOUT>
hipError_t launch_vec_u(const QkParams& p0, int U, hipStream_t s) {
    QkParams p = p0;
    constexpr int RPW = kWave / L;
    p.heads_per_unit = RPW * U;
    p.units_per_token = (p.Q + p.K + p.heads_per_unit - 1) / p.heads_per_unit;
    p.total_units = (uint32_t)(p.T * p.units_per_token);
    p.n_blocks = (p.total_units + 3u) / 4u;
    dim3 grid(p.n_blocks), block(256);
    if (U == 1) hipLaunchKernelGGL((qknorm_rope_vec<DT, L, LAYOUT, 1>), grid, block, 0, s, p);
    else if (U == 2) hipLaunchKernelGGL((qknorm_rope_vec<DT, L, LAYOUT, 2>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((qknorm_rope_vec<DT, L, LAYOUT, 4>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <int DT, int LAYOUT>
hipError_t launch_vec_l(const QkParams& p, int L, int U, hipStream_t s) {
    switch (L) {
    case 4: return launch_vec_u<DT, 4, LAYOUT>(p, U, s);
    case 8: return launch_vec_u<DT, 8, LAYOUT>(p, U, s);
    case 16: return launch_vec_u<DT, 16, LAYOUT>(p, U, s);
    case 32: return launch_vec_u<DT, 32, LAYOUT>(p, U, s);
    default: return launch_vec_u<DT, 64, LAYOUT>(p, U, s);
    }
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
    if (vec) {
        // Steps per wave: one for small launches (latency: spread the rows
        // over as many waves as possible), two once the grid fills the chip.
        const int RPW = kWave / L;
        const int64_t row_steps = a.T * (int64_t)((QK + RPW - 1) / RPW);
        const int U = (row_steps >= 16384) ? 2 : 1;
        const int64_t units = a.T * (int64_t)((QK + RPW * U - 1) / (RPW * U));
        if (units < (int64_t)0xFFFFFF00ll) {
            hipError_t e = (a.layout == 0) ? launch_vec_l<DT, 0>(p, L, U, s)
                                           : launch_vec_l<DT, 1>(p, L, U, s);
            return e;
        }
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
