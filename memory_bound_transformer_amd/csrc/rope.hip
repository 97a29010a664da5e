// rope.hip -- standalone rotary position embedding, in place, for gfx950.
//
// Operation ("thox-edge-ops v2", section 5.1 and requirement R5): the first
// rot_dim channels of every query and key head of token t are rotated by the
// cached angles of position pos[t]; pairs are (i, i + rot/2) for rotate-half
// and (2i, 2i + 1) for interleaved; a position outside [0, max_pos) leaves
// the token untouched (its memory is not written).  Each pair is rotated as
// written -- two rounded products and one rounded sum -- exactly as the fused
// QK-norm prologue rotates it, so norm -> rope reproduces the fused op.
//
// MI355X design: only the rotated span of each head is read and written.  A
// row's rotated chunks (16 bytes each) are a G-lane segment of a wave, G the
// power of two covering them, so 64 / G rows share a wave; the rotate-half
// partner arrives by one lane permute (ds_bpermute), interleaved pairs are
// lane-local.  A scalar kernel covers other shapes and alignments.

#include "mbt_device.hpp"
#include "mbt_launch.hpp"

namespace mbt {
namespace {

struct RopeParams {
    void* q;
    void* k;
    const float* cos_sin;
    const int64_t* pos;
    int64_t max_pos;
    int64_t T;
    int32_t Q, K, D, rot, layout;
    float inv_Q, inv_K;
    uint32_t q_waves, total_waves;
};

__device__ __forceinline__ int32_t token_of(uint32_t r, int heads, float inv_heads) {
    int32_t t = (int32_t)((float)r * inv_heads);
    const int32_t rem = (int32_t)r - t * heads;
    t += (rem >= heads) ? 1 : 0;
    t -= (rem < 0) ? 1 : 0;
    return t;
}

// G lanes per row cover the rotated chunks (rotate-half: 2 * hv of them,
// hv = rot/2 / Vec; interleaved: ceil(rot / Vec)).  The host launches only
// when a cache exists (rot_dim > 0 and max_pos > 0).
//
// Load order as in the fused prologue: the position first, the row's chunk
// beside it, the cos/sin row as soon as the position is in; no load behind a
// lane-dependent branch (lanes past the last row or the rotated span read a
// valid chunk and store nothing -- their stores fall outside the wave's
// buffer range), and an empty asm after each group of loads so the compiler
// does not sink them to their first use.  Spare waves of the last block read
// the last wave's rows and store nothing.
template <int DT, int G, int LAYOUT>
__global__ __launch_bounds__(256) void rope_vec(RopeParams p) {
    constexpr int V = Vec<DT>::n;
    constexpr int RPW = kWave / G;
    constexpr int EB = EltBytes<DT>::n;
    const uint32_t wv0 = (uint32_t)uniform((int)(blockIdx.x * 4u + (threadIdx.x >> 6)));
    const bool spare = wv0 >= p.total_waves;
    const uint32_t wv = spare ? p.total_waves - 1 : wv0;
    const bool is_q = wv < p.q_waves;
    const int heads = is_q ? p.Q : p.K;
    const int64_t nrows = p.T * heads;                      // >= 1: the wave has a row
    const int64_t row0 = (int64_t)(is_q ? wv : wv - p.q_waves) * RPW;
    const int lane = threadIdx.x & 63;
    const int64_t row = row0 + lane / G;
    const bool live = row < nrows;
    const int64_t rowc = live ? row : nrows - 1;
    const int j = lane % G;
    const int half = p.rot >> 1;
    const int hv = half / V;
    const int rc = LAYOUT == 0 ? 2 * hv : (p.rot + V - 1) / V;   // rotated chunks
    const int jc = j < rc ? j : 0;                          // a chunk every lane may read
    const bool is_a = LAYOUT == 0 && jc < hv;
    char* wbase = (char*)(is_q ? p.q : p.k) + row0 * (int64_t)p.D * EB;

    const int64_t ppos = p.pos[token_of((uint32_t)rowc, heads, is_q ? p.inv_Q : p.inv_K)];
    const u32x4 xv = ld16(wbase + (rowc - row0) * (int64_t)p.D * EB + jc * 16);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const bool in_cache = ppos >= 0 && ppos < p.max_pos;
    const float* crow = p.cos_sin + (in_cache ? ppos : 0) * (int64_t)p.rot;
    constexpr int NCS = LAYOUT == 0 ? V / 4 : 1;
    u32x4 cv[NCS], sv[NCS];
    float ci[V / 2], si[V / 2];
    if constexpr (LAYOUT == 0) {
        const int j0 = (is_a ? jc : jc - hv) * V;
#pragma unroll
        for (int i = 0; i < NCS; ++i) {
            cv[i] = ld16(crow + j0 + 4 * i);
            sv[i] = ld16(crow + half + j0 + 4 * i);
        }
    } else {
        const int j0 = jc * (V / 2);
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            const int e = (j0 + i < half) ? j0 + i : 0;
            ci[i] = crow[e];
            si[i] = crow[half + e];
        }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    float a[V], o[V];
    unpack<DT>(xv, a);
    if constexpr (LAYOUT == 0) {
        float b[V];
        unpack<DT>(rot_partner(xv, hv, is_a), b);           // all lanes take part
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float c = __uint_as_float(cv[i / 4][i % 4]);
            const float sn = __uint_as_float(sv[i / 4][i % 4]);
            o[i] = rot_mac(a[i], c, b[i], is_a ? -sn : sn);
        }
    } else {
        const int j0 = jc * (V / 2);
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
            const bool ok = j0 + i < half;                  // past rot_dim: unchanged
            const float r0 = rot_mac(a[2 * i], ci[i], a[2 * i + 1], -si[i]);
            const float r1 = rot_mac(a[2 * i + 1], ci[i], a[2 * i], si[i]);
            o[2 * i] = ok ? r0 : a[2 * i];
            o[2 * i + 1] = ok ? r1 : a[2 * i + 1];
        }
    }
    // written only for a live row, a rotated chunk and a position in the cache
    const bool write = !spare && live && j < rc && in_cache;
    const int64_t wrows = spare ? 0 : (nrows - row0 < RPW) ? nrows - row0 : RPW;
    const __amdgpu_buffer_rsrc_t buf = buf_rsrc(wbase, (uint32_t)(wrows * p.D * EB));
    const uint32_t off = write ? (uint32_t)((row - row0) * p.D * EB + j * 16) : 0xFFFFFFF0u;
    buf_st16(buf, off, pack<DT>(o));
}

// Scalar kernel: one thread per rotated pair of one head-row.
template <int DT>
__global__ __launch_bounds__(256) void rope_scalar(RopeParams p) {
    const int half = p.rot >> 1;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = p.T * (int64_t)(p.Q + p.K);
    if (idx >= rows * half) return;
    const int64_t row = idx / half;
    const int i = (int)(idx % half);
    const int QK = p.Q + p.K;
    const int64_t t = row / QK;
    const int h = (int)(row % QK);
    const int64_t ppos = p.pos[t];
    if (ppos < 0 || ppos >= p.max_pos) return;
    void* x = h < p.Q ? p.q : p.k;
    const int64_t base = h < p.Q ? (t * p.Q + h) * (int64_t)p.D
                                 : (t * p.K + (h - p.Q)) * (int64_t)p.D;
    const int ia = p.layout == 0 ? i : 2 * i;
    const int ib = p.layout == 0 ? i + half : 2 * i + 1;
    const float a = ld_elt<DT>(x, base + ia), b = ld_elt<DT>(x, base + ib);
    const float* crow = p.cos_sin + ppos * (int64_t)p.rot;
    const float c = crow[i], sn = crow[half + i];
    st_elt<DT>(x, base + ia, rot_mac(a, c, b, -sn));
    st_elt<DT>(x, base + ib, rot_mac(b, c, a, sn));
}

template <int DT, int G, int LAYOUT>
hipError_t launch_vec(RopeParams p, hipStream_t s) {
    constexpr int RPW = kWave / G;
    const int64_t qw = (p.T * p.Q + RPW - 1) / RPW;
    const int64_t kw = (p.T * p.K + RPW - 1) / RPW;
    p.q_waves = (uint32_t)qw;
    p.total_waves = (uint32_t)(qw + kw);
    hipLaunchKernelGGL((rope_vec<DT, G, LAYOUT>), dim3((p.total_waves + 3u) / 4u), dim3(256), 0,
                       s, p);
    return hipGetLastError();
}

template <int DT, int LAYOUT>
hipError_t launch_g(const RopeParams& p, int G, hipStream_t s) {
    switch (G) {
    case 2: return launch_vec<DT, 2, LAYOUT>(p, s);
    case 4: return launch_vec<DT, 4, LAYOUT>(p, s);
    case 8: return launch_vec<DT, 8, LAYOUT>(p, s);
    case 16: return launch_vec<DT, 16, LAYOUT>(p, s);
    case 32: return launch_vec<DT, 32, LAYOUT>(p, s);
    default: return launch_vec<DT, 64, LAYOUT>(p, s);
    }
}

template <int DT>
hipError_t launch_dt(const RopeArgs& a, hipStream_t s) {
    constexpr int V = Vec<DT>::n;
    RopeParams p{};
    p.q = a.q; p.k = a.k; p.cos_sin = a.cos_sin; p.pos = a.pos; p.max_pos = a.max_pos;
    p.T = a.T; p.Q = a.Q; p.K = a.K; p.D = a.head_dim; p.rot = a.rot_dim; p.layout = a.layout;
    p.inv_Q = a.Q > 0 ? 1.0f / (float)a.Q : 0.0f;
    p.inv_K = a.K > 0 ? 1.0f / (float)a.K : 0.0f;
    if (a.rot_dim == 0 || a.max_pos == 0) return hipSuccess;      // nothing rotates
    const int half = a.rot_dim / 2, hv = half / V;
    const int rc = a.layout == 0 ? 2 * hv : (a.rot_dim + V - 1) / V;
    int G = 2;
    while (G < rc) G *= 2;
    bool vec = (a.head_dim % V == 0) && G <= kWave && aligned16(a.cos_sin) &&
               (a.Q == 0 || aligned16(a.q)) && (a.K == 0 || aligned16(a.k)) &&
               a.T * (int64_t)(a.Q > a.K ? a.Q : a.K) < (int64_t(1) << 24);
    if (a.layout == 0) vec = vec && (half % V == 0);
    if (vec)
        return a.layout == 0 ? launch_g<DT, 0>(p, G, s) : launch_g<DT, 1>(p, G, s);
    const int64_t n = a.T * (int64_t)(a.Q + a.K) * half;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rope_scalar<DT>), dim3((uint32_t)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
    switch (a.dtype) {
    case kF32: return launch_dt<kF32>(a, s);
    case kF16: return launch_dt<kF16>(a, s);
    default: return launch_dt<kBF16>(a, s);
    }
}

}  // namespace mbt
