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
// The same kernels serve the general forms: token strides (q and k as views
// into a fused QKV buffer; "thox-edge-ops v2", section 6), the single-rounding
// variant (ninfer PR #273, review item 1: rotate the fp32 norm result, round
// once), and the key / value cache write (FlashRT's qkv_split_rope_kvcache;
// "thox-edge-ops v2", section 10): key heads go to row slot[t] of the cache
// and a key wave also copies the token's value heads there.
//
// MI355X design (the pages' CUDA kernel -- one block per token, one warp per
// head, a block barrier between norm and rotation -- is prior art only):
//
//  * A head-row of D elements is a segment of G lanes of one wavefront; each
//    lane holds C 16-byte chunks (8 bf16 / fp16 or 4 fp32) strided by G, so
//    chunk group 0 (channels [0, G * Vec)) contains the whole rotate-half
//    span and only that chunk of each lane takes part in the rotation;
//    interleaved pairs are lane-local, so there any chunk may rotate.
//    G * C * Vec = D.
//    Decode widths use C = 1 (most waves, least work per wave); wider
//    launches take the fewest chunks (2 or 4, where the layout allows) that
//    keep them near one resident round (for D = 256, rot_dim 64 bf16, C = 4:
//    8 lanes x 4 chunks per row, 8 rows per wave).
//  * A wave works on rows of ONE tensor (the q heads, then the k heads, each
//    flattened token-major), so a single set of norm weights sits in its
//    registers and the rows it streams are contiguous in memory.  Each lane
//    finds its row's token with a float reciprocal and one correction.
//  * The sum of squares is a fixed tree: an FMA chain inside each chunk, then
//    a balanced tree over the chunk index -- DPP inside the G-lane segment
//    (gfx950 permlane swaps past 16 lanes), chunk groups combined pairwise.
//    C = 1 and C = 4 therefore give identical bits, so the result does not
//    depend on the batch width, and the standalone norm and rotation entry
//    points reproduce the fused op exactly.  No LDS reduction, no barrier:
//    the normalised value stays in registers between norm and rotation, so
//    in-place calls are safe.
//  * Chunks sit in natural order; the rotate-half partner of chunk j
//    (j + rot/2 / Vec, hv lanes away) arrives by one lane permute
//    (ds_bpermute) per dword.  Interleaved pairs are lane-local.  Each
//    pair is rotated as written -- two rounded products, one rounded sum.
//  * q / k chunks are streamed with nontemporal loads and stores; weights,
//    positions and cos/sin rows use ordinary cached loads.
//  * Workgroups run in dispatch order, round-robin over the 8 XCDs (an
//    XCD-contiguous renumbering measured slower; see the kernel).
//
// A scalar kernel (one wave per head-row, LDS-staged rotation) covers every
// shape and alignment the vector kernel does not; it follows the same
// reduction tree, so both give identical bits.

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
    uint32_t total_waves;     // vector kernel: q_waves + waves over the key rows
};

// The general forms' extra arguments (token strides, slot table, value rows,
// single rounding).  A second kernel argument, so the dense kernel keeps the
// small argument block it measured fastest with at decode widths.
template <bool GEN>
struct QkGen {
    int32_t once;             // 1: rotate the fp32 norm result, round once
    const void* v_in;         // NULL: no value rows
    void* v_out;
    const int64_t* slot;      // NULL: key / value rows of token t go to row t
    int64_t n_slots;          // rows of k_out / v_out when slot != NULL
    int64_t q_in_st, k_in_st, v_in_st, q_out_st, k_out_st, v_out_st;   // token strides
};
template <>
struct QkGen<false> {};

// Output row of token t for a key or value row: slot[t] when a slot table is
// given (-1: not written, e.g. padding), else t.
__device__ __forceinline__ int64_t out_row(const QkGen<true>& g, bool slotted, int64_t t) {
    if (!slotted) return t;
    const int64_t s = g.slot[t];
    return (s >= 0 && s < g.n_slots) ? s : -1;
}

// The V fp32 values of the rotate-half partner lane (hv lanes away).
template <int V>
__device__ __forceinline__ void partner_f32(const float* n, float* nb, int hv, bool is_a) {
#pragma unroll
    for (int h0 = 0; h0 < V; h0 += 4) {
        const u32x4 v{__float_as_uint(n[h0]), __float_as_uint(n[h0 + 1]),
                      __float_as_uint(n[h0 + 2]), __float_as_uint(n[h0 + 3])};
        const u32x4 r = rot_partner(v, hv, is_a);
#pragma unroll
        for (int i = 0; i < 4; ++i) nb[h0 + i] = __uint_as_float(r[i]);
    }
}

// Vector kernel.  DT: dtype; G: lanes per head-row; C: chunks per lane
// (G * C * Vec<DT> = D); LAYOUT: rotary pairing; GEN: false for dense q / k
// with the contract's rounding (the hot path: none of the code below that
// serves the other forms is compiled in), true for token strides, the slot
// table, value rows and the single-rounding flag.  Requires 16-byte aligned
// tensors and token strides, rows of each tensor below 2^24, a 16-byte
// aligned cos/sin cache, and rot/2 a multiple of Vec<DT> with every rotated
// chunk inside chunk group 0 (rotate-half) or rot/2 a multiple of Vec<DT>/2
// and rot a multiple of 4 (interleaved: each chunk's pairs are one aligned
// run of the cache row).  Waves cover the query rows, then the key rows;
// with v_in a key wave also copies the value heads of its rows, unchanged,
// to their slot.
//
// Load order.  The longest dependent chain is position -> cos/sin row, so
// the weights and the position go out first, then the row's chunks, and
// the cos/sin loads follow as soon as the position is in, while the chunks
// are still in flight.  No load sits behind a lane-dependent branch (lanes
// past the last row read zeros (dense form) or that row again (general
// form) and store nothing; lanes outside the rotated span read the first
// cos/sin pairs and ignore them), so each wait the compiler places covers
// only the loads the next step needs.  Measured on MI355X, cold, (Q, K) =
// (24, 4), D = 256, rot_dim 64: with the cos/sin loads behind a wait on the
// row, the gather cost 0.27 us of 3.54 us at T = 256.  The compiler issues
// the weight load ahead of the position; a position read through a buffer
// resource, which it issued ahead of the weights, measured 0.5-0.7 us
// slower at four chunks per lane ((24, 4) T = 512, (16, 2) T = 1024).
//
// ORD, the load order (1 and 2 only with C >= 2; the host picks it from the
// launch's wave count):
//   0  the early order above: at most about ten waves per CU, or a grid
//      that needs several resident rounds;
//   2  the same loads, but the cos/sin loads wait for a block barrier after
//      the reduction: from about ten to twenty waves per CU;
//   1  the whole-block order: no per-lane weight load; the block's two
//      weight rows are staged by all 256 threads behind a block barrier that
//      waits for every load of the block, and the cos/sin loads follow the
//      reduction: from about twenty waves per CU to one full resident round.
// Measured on MI355X, (Q, K) = (24, 4), D = 256, rot_dim 64, cold: T = 512
// (1792 waves) 4.05 / 4.27 / - us for orders 0 / 2 / 1; T = 768 (2688) 5.05
// / 4.97 / 5.39; T = 2048 (7168) 11.8 / 11.6 / 10.2.
template <int DT, int G, int C, int LAYOUT, bool GEN, int ORD>
__global__ __launch_bounds__(256) void qknorm_rope_vec(QkParams p, QkGen<GEN> g) {
    static_assert(ORD == 0 || C >= 2, "orders 1 and 2 stage weights in LDS: C >= 2");
    constexpr bool THR = ORD == 1;
    constexpr int V = Vec<DT>::n;
    constexpr int RPW = kWave / G;     // rows per wave
    constexpr int EB = EltBytes<DT>::n;
    constexpr int L = G * C;           // 16-byte chunks per row
    // C >= 2: the fp32 (w + delta) rows live in LDS rather than in C * V
    // registers per lane: one row per wave (its own tensor's; each wave
    // writes and reads only its own row, so no barrier), or with order 1 the
    // q and k rows once per block, behind a block barrier.
    constexpr int WROWS = C >= 2 ? (THR ? 2 : 4) : 1;
    __shared__ float wsh[WROWS][C >= 2 ? L * V : 1];

    // Blocks keep their dispatch order, which deals them round-robin over
    // the 8 XCDs.  Renumbering them so that each XCD takes a contiguous range
    // of rows was measured slower at every width, and badly so when key
    // waves carry value heads (twice a query wave's bytes): a contiguous
    // range put those on one XCD, whose share of the fabric then bounded the
    // launch (15.2 us against 11.9 us, (Q, K) = (24, 4), T = 2048).
    // Spare waves of the last block do not leave early (an exit test first
    // would put a round trip for that one argument ahead of all others):
    // they read the last wave's rows and store nothing.
    const uint32_t wv0 = (uint32_t)uniform((int)(blockIdx.x * 4u + (threadIdx.x >> 6)));
    if constexpr (GEN) {
        // Every argument is needed up front: an empty asm that takes them
        // makes the compiler fetch them in one batch, not in further
        // dependent rounds inside the branches below.
        asm volatile("" ::"s"(g.v_in), "s"(g.v_in_st), "s"(g.slot), "s"(g.n_slots),
                     "s"(g.v_out), "s"(g.v_out_st), "s"(g.q_in_st), "s"(g.k_in_st),
                     "s"(g.q_out_st), "s"(g.k_out_st), "s"(g.once), "s"(p.q_in), "s"(p.k_in),
                     "s"(p.q_out), "s"(p.k_out), "s"(p.w_q), "s"(p.w_k), "s"(p.pos),
                     "s"(p.cos_sin));
    }
    const bool spare = wv0 >= p.total_waves;
    const uint32_t wv = spare ? p.total_waves - 1 : wv0;
    const bool is_q = wv < p.q_waves;                       // wave-uniform tensor
    const int heads = is_q ? p.Q : p.K;
    const float inv_heads = is_q ? p.inv_Q : p.inv_K;
    const int64_t nrows = p.T * heads;                      // >= 1: the wave has a row
    const int64_t row0 = (int64_t)(is_q ? wv : wv - p.q_waves) * RPW;
    const char* src = (const char*)(is_q ? p.q_in : p.k_in);
    char* dst = (char*)(is_q ? p.q_out : p.k_out);
    const char* wp = (const char*)(is_q ? p.w_q : p.w_k);

    const int lane = threadIdx.x & 63;
    const int j = lane % G;                                 // lane within the row
    const int64_t row = row0 + lane / G;
    const bool live = row < nrows;
    const int64_t rowc = live ? row : nrows - 1;            // a row every lane may read
    const int half = p.rot >> 1;
    const int hv = half / V;                                // rotate-half: chunks per half
    const bool is_a = LAYOUT == 0 && j < hv;
    const bool is_b = LAYOUT == 0 && j >= hv && j < 2 * hv;

    // The row's token t and head h: a float reciprocal and one correction.
    const uint32_t r32 = (uint32_t)rowc;
    int32_t t = (int32_t)((float)r32 * inv_heads);
    int32_t h = (int32_t)r32 - t * heads;
    if (h >= heads) { t += 1; h -= heads; }
    if (h < 0) { t -= 1; h += heads; }

    // ---- loads ----
    // Order: position, weights, the row's chunks; then, once the position
    // is in, the cos/sin row.  GEN puts its loads behind wave-uniform
    // branches (value rows, slot) first: vmcnt retires loads in issue order,
    // and a conditional load issued after the position would leave the
    // compiler a conservative wait there.  A key wave that carries value
    // rows therefore issues its cos/sin loads when those rows are in (as
    // early as a wait on its own chunks would allow), and stores them at
    // once, so they are not held in registers through the arithmetic.
    u32x4 vx[GEN ? C : 1];
    bool carry_v = false, slotted = false;
    int64_t slot_raw = t;                                   // key / value output row (raw)
    // The position-independent parts of the cos/sin addresses, formed
    // before any load.  Without a table (rot_dim 0 or an empty cache) every
    // lane reads the first V floats of the weight row (at least 64 bytes)
    // instead, and nothing uses them.
    const bool table = p.rot > 0 && p.max_pos > 0;          // wave-uniform
    const float* cs_base = table ? p.cos_sin : (const float*)wp;
    const int hoff = table ? half : 0;                      // sin half of the row
    const int cs_j0 = LAYOUT == 0 ? (table ? (is_a ? j : (is_b ? j - hv : 0)) * V : 0)
                                  : j * (V / 2);            // first pair (chunk group 0)
    if constexpr (GEN) {
        // value rows: a key wave also carries the value heads of its rows
        // (adjacent to the key heads in a fused QKV buffer)
        carry_v = !is_q && g.v_in != nullptr;               // wave-uniform
        if (carry_v) {
            const char* vsrc =
                (const char*)g.v_in + ((int64_t)t * g.v_in_st + (int64_t)h * p.D) * EB;
#pragma unroll
            for (int k = 0; k < C; ++k) vx[k] = ld16_nt(vsrc + (k * G + j) * 16);
        }
        slotted = !is_q && g.slot != nullptr;               // wave-uniform
        if (slotted) slot_raw = g.slot[t];
    }
    // the head of the longest chain: position -> cos/sin row
    const int64_t ppos = p.pos[t];
    // weights: chunk (lane mod L) of the tensor's row -- for C = 1 that is
    // the lane's own chunk, for C >= 2 the staging share of its LDS row;
    // order 1 stages both rows block-wide instead
    u32x4 wraw{0u, 0u, 0u, 0u};
    if constexpr (!THR) wraw = ld16(wp + (lane % L) * 16);
    // the row's chunks: dense rows through a buffer over the wave's rows (a
    // scalar base and 32-bit lane offsets, no per-lane 64-bit address
    // arithmetic; lanes past the last row read zeros, and their results are
    // not stored); the general form at its own token and head strides
    u32x4 x[C];
    const uint32_t rofs = (uint32_t)((lane / G) * p.D * EB);   // the lane's row in the wave
    if constexpr (GEN) {
        const char* xsrc =
            src + ((int64_t)t * (is_q ? g.q_in_st : g.k_in_st) + (int64_t)h * p.D) * EB;
#pragma unroll
        for (int k = 0; k < C; ++k) x[k] = ld16_nt(xsrc + (k * G + j) * 16);
    } else {
        const int64_t lrows = (nrows - row0 < RPW) ? nrows - row0 : RPW;   // >= 1
        const __amdgpu_buffer_rsrc_t wsrc =
            buf_rsrc((void*)(src + row0 * (int64_t)p.D * EB), (uint32_t)(lrows * p.D * EB));
#pragma unroll
        for (int k = 0; k < C; ++k) x[k] = buf_ld16_nt(wsrc, rofs + (uint32_t)((k * G + j) * 16));
    }
    // An empty asm that may touch memory: the loads above cannot be moved
    // below it (to their first use), and it emits no instruction or wait.
    // The sched_barrier keeps arithmetic on their results (the position
    // test) from being hoisted above them.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // cos/sin of the position (raw bits; decoded where the rotation uses them)
    const bool rotate = (ppos >= 0) && (ppos < p.max_pos) && (p.rot > 0);
    constexpr int NCS = LAYOUT == 0 ? V / 4 : 1;
    u32x4 cs_c4[NCS], cs_s4[NCS];
    // interleaved: every chunk group may hold rotated pairs (they are
    // lane-local), so each of the C chunks has its own cos / sin run
    constexpr int NCK = LAYOUT == 1 ? C : 1;
    float cs_c[NCK][V / 2], cs_s[NCK][V / 2];
    bool lane_rot = false;                                  // rotate-half (group 0)
    bool rot_k[NCK];                                        // interleaved, per chunk
    // (Not behind a branch, which the compiler would sink the loads into.)
    const float* crow = cs_base + (rotate ? ppos : 0) * (int64_t)p.rot;
    // Interleaved, chunk k: its V/2 consecutive pairs are all below rot/2 or
    // all past it (the host requires rot/2 to be a multiple of V/2), read as
    // one 16-byte (8-byte for fp32) run of cos and one of sin; chunks past
    // rot/2 read the first run and keep R(n).
    auto load_cs_chunk = [&](int k) {
        const int j0 = cs_j0 + k * G * (V / 2);
        rot_k[k] = rotate && (j0 < half);
        const int e0 = (table && j0 < half) ? j0 : 0;
        if constexpr (V == 8) {
            const u32x4 cv = ld16(crow + e0), sv = ld16(crow + hoff + e0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs_c[k][i] = __uint_as_float(cv[i]);
                cs_s[k][i] = __uint_as_float(sv[i]);
            }
        } else {
            const u32x2 cv = *reinterpret_cast<const u32x2*>(crow + e0);
            const u32x2 sv = *reinterpret_cast<const u32x2*>(crow + hoff + e0);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                cs_c[k][i] = __uint_as_float(cv[i]);
                cs_s[k][i] = __uint_as_float(sv[i]);
            }
        }
    };
    // Interleaved rows in order 1 issue a chunk's runs two chunks ahead of
    // its rotation, not all C up front: with C = 4 that is 16 live registers
    // of cos/sin instead of 32, which keeps the kernel at eight waves per
    // SIMD (63 VGPRs for bf16, against 83 and five waves up front).  Order 1
    // serves launches of up to one round at eight waves per SIMD, so at five
    // its last waves waited for a second round: (Q, K) = (24, 4), T = 2048,
    // rot_dim 256, cold, 13.07 -> 10.72 us on MI355X.  The lower orders fit
    // in one round at five waves per SIMD and keep every run up front (2 %
    // faster at (16, 2), T = 2048).
    constexpr int PIPE = (LAYOUT == 1 && ORD == 1) ? 2 : C;   // runs issued up front
    auto load_cs = [&]() {
        if constexpr (LAYOUT == 0) {
            lane_rot = rotate && (is_a || is_b);
            const int j0 = cs_j0;
#pragma unroll
            for (int i = 0; i < NCS; ++i) {
                cs_c4[i] = ld16(crow + j0 + 4 * i);
                cs_s4[i] = ld16(crow + hoff + j0 + 4 * i);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NCK && k < PIPE; ++k) load_cs_chunk(k);
        }
    };
    if constexpr (ORD == 0) {
        // sched_barrier: no arithmetic on the row is hoisted above these loads
        __builtin_amdgcn_sched_barrier(0);
        load_cs();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);                  // all loads issued
    }

    // ---- C >= 2: stage (w + delta) in LDS ----
    const float* wrow = nullptr;
    if constexpr (C >= 2 && !THR) {                         // the wave's own row
        const int wib = threadIdx.x >> 6;
        if (lane < L) {
            float wf[V];
            unpack<DT>(wraw, wf);
#pragma unroll
            for (int i = 0; i < V; ++i) wsh[wib][lane * V + i] = wf[i] + p.delta;
        }
        __builtin_amdgcn_wave_barrier();
        wrow = wsh[wib];
    }
    if constexpr (THR) {                                    // both rows, block-wide
        // Every lane loads one element of w_q, waits, then one of w_k: two
        // dependent round trips before the barrier, as measured best on
        // MI355X at (Q, K) = (24, 4), T = 2048.  Both loads behind one wait,
        // 16-byte loads on the first 2 L lanes, or a third dependent load
        // were 9-12 % / 11-12 % / 1-2 % slower (the same bits).
        for (int i = threadIdx.x; i < p.D; i += 256) {
            wsh[0][i] = (p.Q > 0) ? ld_elt<DT>(p.w_q, i) + p.delta : 0.0f;
            wsh[1][i] = (p.K > 0) ? ld_elt<DT>(p.w_k, i) + p.delta : 0.0f;
        }
        __syncthreads();                                    // after every load of the block
        wrow = wsh[is_q ? 0 : 1];
    }

    // ---- output rows ----
    int64_t orow = t;
    if constexpr (GEN)
        if (slotted) orow = (slot_raw >= 0 && slot_raw < g.n_slots) ? slot_raw : -1;
    const bool keep = !spare && orow >= 0;
    int64_t out_off = rowc * p.D;
    if constexpr (GEN)
        out_off = (keep ? orow : 0) * (is_q ? g.q_out_st : g.k_out_st) + (int64_t)h * p.D;
    if constexpr (GEN) {
        if (carry_v && keep) {                              // value heads: copy to the slot
            char* vdst = (char*)g.v_out + (orow * g.v_out_st + (int64_t)h * p.D) * EB;
#pragma unroll
            for (int k = 0; k < C; ++k) st16_nt(vdst + (k * G + j) * 16, vx[k]);
        }
    }

    // ---- sum of squares: chunk chains, G-lane tree, groups pairwise ----
    float part[C];
#pragma unroll
    for (int k = 0; k < C; ++k) {
        float f[V];
        unpack<DT>(x[k], f);
        part[k] = seg_sum<G>(chunk_sumsq<DT>(f));
    }
    float ss;
    if constexpr (C == 1) ss = part[0];
    else if constexpr (C == 2) ss = part[0] + part[1];
    else ss = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = inv_rms(ss, p.inv_D, p.eps);
    if constexpr (ORD == 1) load_cs();
    if constexpr (ORD == 2) {
        __syncthreads();                                    // every row of the block summed
        load_cs();
    }

    // ---- normalise, round, rotate (group 0 only), store ----
    float wreg[C >= 2 ? 1 : V];
    if constexpr (C == 1) {
        unpack<DT>(wraw, wreg);
#pragma unroll
        for (int i = 0; i < V; ++i) wreg[i] += p.delta;
    }
    char* rdst = dst + out_off * EB;
    // dense form: the wave's rows as one buffer (its rows below nrows; none
    // for a spare wave)
    const int64_t wrows = spare ? 0 : (nrows - row0 < RPW) ? nrows - row0 : RPW;
    const __amdgpu_buffer_rsrc_t wdst =
        buf_rsrc(dst + row0 * (int64_t)p.D * EB, (uint32_t)(wrows * p.D * EB));
#pragma unroll
    for (int k = 0; k < C; ++k) {
        float f[V], n[V];
        unpack<DT>(x[k], f);                                // decoded again: fewer live VGPRs
        if constexpr (C >= 2) {
            const float* wk = wrow + (k * G + j) * V;
#pragma unroll
            for (int i = 0; i < V; ++i) n[i] = (f[i] * inv) * wk[i];
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) n[i] = (f[i] * inv) * wreg[i];
        }
        u32x4 out = pack<DT>(n);                            // R(n): the rounded value
        if (LAYOUT == 1 || k == 0) {
            // the rotation's inputs: R(n) (the contract) or n itself (once)
            bool once = false;
            if constexpr (GEN) once = g.once != 0;
            float a[V], o[V];
            if (once) {
#pragma unroll
                for (int i = 0; i < V; ++i) a[i] = n[i];
            } else {
                unpack<DT>(out, a);
            }
            if constexpr (LAYOUT == 0) {
                float b[V];
                if (once) {
                    partner_f32<V>(n, b, hv, is_a);
                } else {
                    unpack<DT>(rot_partner(out, hv, is_a), b);
                }
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const float c = __uint_as_float(cs_c4[i / 4][i % 4]);
                    const float s = __uint_as_float(cs_s4[i / 4][i % 4]);
                    // o = own * c + partner * s', s' = -s for the first half
                    o[i] = rot_mac(a[i], c, b[i], is_a ? -s : s);
                }
            } else {
                const int kk = LAYOUT == 1 ? k : 0;
#pragma unroll
                for (int i = 0; i < V / 2; ++i) {
                    o[2 * i] = rot_mac(a[2 * i], cs_c[kk][i], a[2 * i + 1], -cs_s[kk][i]);
                    o[2 * i + 1] = rot_mac(a[2 * i + 1], cs_c[kk][i], a[2 * i], cs_s[kk][i]);
                }
            }
            // every lane computes the rotation (no branch, so the cos/sin
            // loads stay where they were issued); lanes outside the rotated
            // span, and tokens outside the cache, keep R(n)
            const bool take = LAYOUT == 1 ? rot_k[LAYOUT == 1 ? k : 0] : lane_rot;
            const u32x4 ro = pack<DT>(o);
#pragma unroll
            for (int d = 0; d < 4; ++d) out[d] = take ? ro[d] : out[d];
        }
        if constexpr (PIPE < C) {
            // the runs PIPE chunks on, issued once this chunk's are used
            if (k + PIPE < C) {
                __builtin_amdgcn_sched_barrier(0);
                load_cs_chunk(k + PIPE);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (GEN) {
            if (keep) st16_nt(rdst + (k * G + j) * 16, out);
        } else {
            // through the wave's buffer: lanes past the last row fall outside
            // it and are dropped, with no branch for the code above to sink into
            buf_st16_nt(wdst, rofs + (uint32_t)((k * G + j) * 16), out);
        }
    }
}

// Scalar kernel: any D <= 512, any even rot, element-aligned pointers and
// strides.  One wave per head-row (4 rows per 256-thread block); a token's
// rows are its Q query heads, its K key heads, then (with v_in) its K value
// heads, which are copied to their slot.  Lane c owns chunk c (Vec<DT>
// consecutive elements; lane c + 64 too for fp32 rows past 256), so the sum
// of squares follows the vector kernels' tree (zero lanes add nothing); the
// normalised row (rounded, or not for the single-rounding variant) is staged
// in LDS for the rotation.
template <int DT>
__global__ __launch_bounds__(256) void qknorm_rope_scalar(QkParams p, QkGen<true> g) {
    constexpr int V = Vec<DT>::n;
    constexpr int CPL = (512 / V + kWave - 1) / kWave;      // chunks per lane
    __shared__ float stage[4][512];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + w;
    const int per_t = p.Q + p.K + (g.v_in ? p.K : 0);
    const int64_t rows = p.T * per_t;
    const bool live = row < rows;
    const int64_t t = live ? row / per_t : 0;
    const int hh = live ? (int)(row % per_t) : 0;
    const int kind = hh < p.Q ? 0 : (hh < p.Q + p.K ? 1 : 2);
    const int h = kind == 0 ? hh : (kind == 1 ? hh - p.Q : hh - p.Q - p.K);
    const void* src = kind == 0 ? p.q_in : kind == 1 ? p.k_in : g.v_in;
    void* dst = kind == 0 ? p.q_out : kind == 1 ? p.k_out : g.v_out;
    const int64_t in_st = kind == 0 ? g.q_in_st : kind == 1 ? g.k_in_st : g.v_in_st;
    const int64_t out_st = kind == 0 ? g.q_out_st : kind == 1 ? g.k_out_st : g.v_out_st;
    const void* wp = kind == 0 ? p.w_q : p.w_k;
    const int64_t ibase = t * in_st + (int64_t)h * p.D;
    const int64_t orow = live ? out_row(g, kind != 0 && g.slot != nullptr, t) : -1;
    const int64_t obase = (orow >= 0 ? orow : 0) * out_st + (int64_t)h * p.D;
    float f[CPL][V];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = lane + k * kWave;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int e = c * V + i;
            f[k][i] = (live && e < p.D) ? ld_elt<DT>(src, ibase + e) : 0.0f;
        }
        // 64-chunk groups reduce on their own, then add: the canonical tree
        const float part = seg_sum<64>(chunk_sumsq<DT>(f[k]));
        ss = (k == 0) ? part : ss + part;
    }
    const float inv = inv_rms(ss, p.inv_D, p.eps);
    if (kind != 2) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int e = (lane + k * kWave) * V + i;
                if (live && e < p.D) {
                    const float n = (f[k][i] * inv) * (ld_elt<DT>(wp, e) + p.delta);
                    stage[w][e] = g.once ? n : round_trip<DT>(n);
                }
            }
        }
    }
    __syncthreads();
    if (!live || orow < 0) return;
    if (kind == 2) {                                       // value row: copy the bits
        for (int e = lane; e < p.D; e += kWave) {
            if constexpr (DT == kF32)
                reinterpret_cast<uint32_t*>(dst)[obase + e] =
                    reinterpret_cast<const uint32_t*>(src)[ibase + e];
            else
                reinterpret_cast<uint16_t*>(dst)[obase + e] =
                    reinterpret_cast<const uint16_t*>(src)[ibase + e];
        }
        return;
    }
    const int64_t ppos = p.pos[t];
    const bool rotate = (ppos >= 0) && (ppos < p.max_pos) && (p.rot > 0);
    const int half = p.rot >> 1;
    const float* cs = p.cos_sin + (rotate ? ppos * (int64_t)p.rot : 0);
    for (int e = lane; e < p.D; e += kWave) {
        float o = stage[w][e];
        if (rotate && e < p.rot) {
            int jj, a, b;
            if (p.layout == 0) {                     // rotate-half
                jj = (e < half) ? e : e - half;
                a = jj;
                b = jj + half;
            } else {                                 // interleaved
                jj = e >> 1;
                a = 2 * jj;
                b = 2 * jj + 1;
            }
            const float c = cs[jj], s = cs[half + jj];
            o = (e == a) ? rot_mac(stage[w][a], c, stage[w][b], -s)
                         : rot_mac(stage[w][b], c, stage[w][a], s);
        }
        st_elt<DT>(dst, obase + e, o);
    }
}

// Chunks per lane: the fewest that bring the launch to at most kCWaves
// waves (about ten per CU: one resident round, short per-wave work), and at
// most kCMax.  Launch-shape thresholds are compile-time constants, the
// measured best on MI355X; every shape gives the same bits.
constexpr int64_t kCWaves = 2560;
// Interleaved pairs rotate in every chunk, so a lane's chain grows with its
// chunks: those launches keep fewer chunks per lane, up to this many waves
// (one chunk per lane only up to kCWavesInterleaved1).
constexpr int64_t kCWavesInterleaved = 8000;
constexpr int64_t kCWavesInterleaved1 = 6000;
constexpr int kCMax = 4;

// Waves of a launch with G lanes per row.
int64_t vec_waves(const QkParams& p, int G) {
    const int rpw = kWave / G;
    return (p.T * p.Q + rpw - 1) / rpw + (p.T * p.K + rpw - 1) / rpw;
}

// Load orders by wave count (C >= 2): order 2 above kMidWavesLo waves,
// order 1 above kThrWavesLo, both up to kThrWavesHi (one full resident
// round of 256 CUs x 4 SIMDs x 8 waves); order 0 elsewhere.
constexpr int64_t kMidWavesLo = 2560;
constexpr int64_t kThrWavesLo = 5000;
constexpr int64_t kThrWavesHi = 8192;

template <int DT, int G, int C, int LAYOUT, bool GEN, int ORD>
hipError_t launch_vec(const QkParams& p0, const QkGen<true>& g0, hipStream_t s) {
    QkParams p = p0;
    constexpr int RPW = kWave / G;
    const int64_t qw = (p.T * p.Q + RPW - 1) / RPW;
    const int64_t kw = (p.T * p.K + RPW - 1) / RPW;
    if (qw + kw > 0x7FFFFFFFll) return hipErrorInvalidValue;
    p.q_waves = (uint32_t)qw;
    p.total_waves = (uint32_t)(qw + kw);
    const uint32_t n_blocks = (p.total_waves + 3u) / 4u;
    QkGen<GEN> g{};
    if constexpr (GEN) g = g0;
    hipLaunchKernelGGL((qknorm_rope_vec<DT, G, C, LAYOUT, GEN, ORD>), dim3(n_blocks), dim3(256),
                       0, s, p, g);
    return hipGetLastError();
}

// (G, C) with G * C = L lanes-of-chunks per row; G a power of two >= 4.
template <int DT, int LAYOUT, bool GEN>
hipError_t launch_gc(const QkParams& p, const QkGen<true>& g, int L, int C, hipStream_t s) {
    int ord = 0;
    if (C >= 2) {
        const int64_t w = vec_waves(p, L / C);
        if (w <= kThrWavesHi) ord = w > kThrWavesLo ? 1 : (w > kMidWavesLo ? 2 : 0);
    }
#define MBT_QK_CASE1(LL)                                                 \
    if (L == LL && C == 1) return launch_vec<DT, LL, 1, LAYOUT, GEN, 0>(p, g, s);
#define MBT_QK_CASE(LL, CC)                                              \
    if (L == LL && C == CC)                                              \
        return ord == 1   ? launch_vec<DT, LL / CC, CC, LAYOUT, GEN, 1>(p, g, s)   \
               : ord == 2 ? launch_vec<DT, LL / CC, CC, LAYOUT, GEN, 2>(p, g, s)   \
                          : launch_vec<DT, LL / CC, CC, LAYOUT, GEN, 0>(p, g, s);
    MBT_QK_CASE1(4)
    MBT_QK_CASE1(8) MBT_QK_CASE(8, 2)
    MBT_QK_CASE1(16) MBT_QK_CASE(16, 2) MBT_QK_CASE(16, 4)
    MBT_QK_CASE1(32) MBT_QK_CASE(32, 2) MBT_QK_CASE(32, 4)
    MBT_QK_CASE1(64) MBT_QK_CASE(64, 2) MBT_QK_CASE(64, 4)
#undef MBT_QK_CASE
#undef MBT_QK_CASE1
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const QkArgs& a, hipStream_t s) {
    constexpr int V = Vec<DT>::n;
    constexpr int EB = EltBytes<DT>::n;
    QkParams p{};
    p.q_in = a.q_in; p.k_in = a.k_in; p.q_out = a.q_out; p.k_out = a.k_out;
    p.w_q = a.w_q; p.w_k = a.w_k; p.cos_sin = a.cos_sin; p.pos = a.pos;
    QkGen<true> g{};
    g.v_in = a.v_in; g.v_out = a.v_out; g.slot = a.slot; g.n_slots = a.n_slots;
    g.q_in_st = a.q_in_stride; g.k_in_st = a.k_in_stride; g.v_in_st = a.v_in_stride;
    g.q_out_st = a.q_out_stride; g.k_out_st = a.k_out_stride; g.v_out_st = a.v_out_stride;
    g.once = a.round_once ? 1 : 0;
    p.max_pos = a.max_pos; p.T = a.T; p.Q = a.Q; p.K = a.K; p.D = a.head_dim;
    p.rot = a.rot_dim; p.eps = a.eps; p.inv_D = 1.0f / (float)a.head_dim;
    p.delta = (float)a.weight_offset;
    p.layout = a.layout;

    // Vector path conditions: 16-byte chunks everywhere, rows of each tensor
    // below 2^24 (the token index uses a float reciprocal).
    auto st16 = [](int64_t st) { return (st * EB) % 16 == 0; };
    const int L = a.head_dim / V;
    bool vec = (a.head_dim % V == 0) && (L == 4 || L == 8 || L == 16 || L == 32 || L == 64);
    if (a.Q > 0)
        vec = vec && aligned16(a.q_in) && aligned16(a.q_out) && aligned16(a.w_q) &&
              st16(a.q_in_stride) && st16(a.q_out_stride);
    if (a.K > 0)
        vec = vec && aligned16(a.k_in) && aligned16(a.k_out) && aligned16(a.w_k) &&
              st16(a.k_in_stride) && st16(a.k_out_stride);
    if (a.v_in)
        vec = vec && aligned16(a.v_in) && aligned16(a.v_out) && st16(a.v_in_stride) &&
              st16(a.v_out_stride);
    if (a.rot_dim > 0 && a.max_pos > 0) {
        // rotate-half: rot/2 a multiple of Vec; interleaved: of Vec/2, with
        // 16-byte runs of the cache (rows of a multiple of 4 floats)
        vec = vec && aligned16(a.cos_sin);
        if (a.layout == 0) vec = vec && ((a.rot_dim / 2) % V == 0);
        else vec = vec && ((a.rot_dim / 2) % (V / 2) == 0) && (a.rot_dim % 4 == 0);
    }
    const int QK = a.Q + a.K;
    vec = vec && a.T * (int64_t)(a.Q > a.K ? a.Q : a.K) < (int64_t(1) << 24);
    if (vec) {
        // Chunks per lane: the fewest (1, 2, 4) whose launch has at most
        // kCWaves waves (kCWavesInterleaved for interleaved pairs), else the
        // most allowed.  Rotate-half rotates chunk group 0 only (its partner
        // permute spans G lanes), so G must cover the rotated chunks;
        // interleaved pairs are lane-local, so any chunk may rotate.
        // Measured on MI355X, cold, D = 256: rotate-half rot_dim 64 (24, 4)
        // T = 256 takes 2 (3.29 us; 1 chunk 3.43, 4 chunks 3.37), T = 512
        // takes 4, and bounds of 1500, 4000 or 8000 waves were slower or
        // equal at every configuration-3 width; interleaved full rotary
        // with the 8000 bound against 2560: (24, 4) T = 256 / 512 / 1024 /
        // 2048 3.35 / 4.48 / 6.57 / 11.32 -> 3.26 / 4.37 / 6.43 / 11.14 us,
        // (16, 2) T = 512 / 1024 / 2048 3.66 / 5.28 / 7.94 -> 3.60 / 4.94 /
        // 7.83 us.  One chunk per lane only up to 6000 of those waves: (24, 4)
        // T = 512 (7168 waves at one chunk, 3584 at two) 4.43 -> 4.26 us,
        // every other configuration-3 cell unchanged; a single bound of
        // 4000 also took T = 1024 to four chunks (6.44 -> 6.58 us).
        const int half = a.rot_dim / 2;
        const int rc = (a.rot_dim == 0) ? 0
                       : (a.layout == 0 ? 2 * (half / V) : (a.rot_dim + V - 1) / V);
        int C = 1;
        const int64_t cwaves = a.layout == 0 ? kCWaves : kCWavesInterleaved;
        const int64_t c1waves = a.layout == 0 ? kCWaves : kCWavesInterleaved1;
        if (vec_waves(p, L) > c1waves) {
            for (int cand : {2, 4}) {
                const int G = L / cand;
                if (cand > kCMax || G < 4 || (a.layout == 0 && G < rc)) continue;
                C = cand;
                if (vec_waves(p, G) <= cwaves) break;
            }
        }
        p.inv_Q = a.Q > 0 ? 1.0f / (float)a.Q : 0.0f;
        p.inv_K = a.K > 0 ? 1.0f / (float)a.K : 0.0f;
        // the general kernel only where a stride, slot, value row or the
        // single-rounding flag asks for it
        const int64_t qrow = (int64_t)a.Q * a.head_dim, krow = (int64_t)a.K * a.head_dim;
        const bool gen = a.round_once || a.slot || a.v_in ||
                         (a.Q > 0 && (a.q_in_stride != qrow || a.q_out_stride != qrow)) ||
                         (a.K > 0 && (a.k_in_stride != krow || a.k_out_stride != krow));
        auto run = [&](const QkParams& pp) {
            if (gen)
                return (a.layout == 0) ? launch_gc<DT, 0, true>(pp, g, L, C, s)
                                       : launch_gc<DT, 1, true>(pp, g, L, C, s);
            return (a.layout == 0) ? launch_gc<DT, 0, false>(pp, g, L, C, s)
                                   : launch_gc<DT, 1, false>(pp, g, L, C, s);
        };
        // A launch without a slot table or value rows, of more than one
        // resident round but at most one and a half (8192 < waves <= 12288),
        // whose second round would run half empty, runs as two launches over
        // the two halves of the tokens, each within one round (the same
        // bits: every row is computed alone).  Measured on MI355X, cold, D = 256 rot_dim 64 bf16, on
        // three machines: (16, 2) T = 4096 (9216 waves) 4.6-5.6 % faster on
        // each, (24, 4) T = 3072 (10752) 2.7-3.3 %, (16, 2) T = 5120
        // (11520) 2.5-4.6 %; from about 12500 waves the split was neither
        // reliably faster nor slower ((24, 4) T = 4096: -4.0 / +3.9 /
        // -0.9 %), and two launches of more than a round each were slower
        // ((16, 2) T = 8192: 26.4 -> 29.6 us).  q and k as strided views of a
        // fused QKV buffer gain alike (2.0-4.0 % at the same widths); the
        // KV-cache form, whose key waves also carry the value heads, was
        // mixed (+11.6 % at (16, 2) T = 4096, -4.8 / -6.3 % at the others)
        // and keeps one launch.
        const int64_t w = vec_waves(p, L / C);
        if (!a.slot && !a.v_in && w > kThrWavesHi && w <= kThrWavesHi + kThrWavesHi / 2 &&
            a.T >= 2) {
            const int64_t T1 = (a.T + 1) / 2;
            QkParams p2 = p;
            p.T = T1;
            p2.T = a.T - T1;
            if (a.Q > 0) {
                p2.q_in = (const char*)a.q_in + T1 * a.q_in_stride * EB;
                p2.q_out = (char*)a.q_out + T1 * a.q_out_stride * EB;
            }
            if (a.K > 0) {
                p2.k_in = (const char*)a.k_in + T1 * a.k_in_stride * EB;
                p2.k_out = (char*)a.k_out + T1 * a.k_out_stride * EB;
            }
            p2.pos = a.pos + T1;
            const hipError_t e = run(p);
            if (e != hipSuccess) return e;
            return run(p2);
        }
        return run(p);
    }
    const int64_t blocks = (a.T * (int64_t)(QK + (a.v_in ? a.K : 0)) + 3) / 4;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qknorm_rope_scalar<DT>), dim3((uint32_t)blocks), dim3(256), 0, s, p, g);
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
