/*
 * abi_roundtrip.c -- libmbt driven from plain C, with no Python and no
 * PyTorch: device buffers from hipMalloc, the null stream, results copied
 * back and checked against the CPU oracle (liboracle, test infrastructure).
 *
 * Cases: the fused QK-RMSNorm + RoPE prologue ("thox-edge-ops v2", section
 * 5.1; tokens inside and outside the cos/sin cache), the same on a fused
 * QKV buffer with the key / value cache write (FlashRT's decoder kernel
 * list, qkv_split_rope_kvcache; a padding slot), the residual-add
 * RMSNorm to static FP8 (FlashRT "optimization details", fused kernel
 * table) with its in-place residual update, the gated SiLU activation, the
 * standalone rotation (interleaved pairs, in place, bit for bit), the
 * adaptive norm to FP8 with its calibration pass, and one rejected call.  The comparison rules are the parity suite's: <= 1 bf16
 * ulp for normalised, rotated and activated values (a rotated value may
 * also move by the rotation of a one-ulp difference in its inputs), FP8
 * codes within one step, residual sums bit-identical.
 *
 * Exit status 0: every check passed.  Each case prints one line first.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mbt.h"
#include "mbt_oracle.h"

static int failures = 0;

#define HIP_OK(call)                                                          \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), \
                    __FILE__, __LINE__);                                      \
            exit(2);                                                          \
        }                                                                     \
    } while (0)

static void check(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

/* A fixed stream of roughly normal values: sums of four uniforms from a
 * 64-bit linear congruential generator, scaled to standard deviation sd. */
static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 11) * (1.0 / 9007199254740992.0);
}
static float normalish(double mean, double sd) {
    double s = uniform01() + uniform01() + uniform01() + uniform01() - 2.0;
    return (float)(mean + sd * s * 1.7320508075688772);  /* var(sum) = 1/3 */
}

static uint16_t* bf16_array(size_t n, double mean, double sd) {
    uint16_t* a = malloc(n * sizeof *a);
    for (size_t i = 0; i < n; ++i) a[i] = mbt_ref_f32_to_bf16(normalish(mean, sd));
    return a;
}

/* A device buffer of `bytes`, holding a copy of `host` (or uninitialised
 * when host is NULL: an output). */
static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    if (host && bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void from_device(void* host, const void* dev, size_t bytes) {
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
}

/* bf16 patterns on a monotone integer line (+0 and -0 coincide). */
static int64_t ordered(uint16_t h) {
    return (h & 0x8000) ? -(int64_t)(h & 0x7FFF) : (int64_t)(h & 0x7FFF);
}
static int64_t ulp_dist(uint16_t a, uint16_t b) {
    int64_t d = ordered(a) - ordered(b);
    return d < 0 ? -d : d;
}
static double bf16_spacing(uint16_t h) {
    int e = (h >> 7) & 0xFF;
    return ldexp(1.0, (e > 0 ? e : 1) - 127 - 7);
}

/* ---- the prologue ------------------------------------------------------- */
static void case_prologue(void) {
    enum { T = 6, Q = 4, K = 2, D = 128, ROT = 64, MAXPOS = 64 };
    const float eps = 1e-6f;
    const int32_t delta = 1;
    printf("case prologue: T=%d Q=%d K=%d D=%d rot=%d bf16, rotate-half\n", T, Q, K, D, ROT);
    fflush(stdout);
    uint16_t* q = bf16_array((size_t)T * Q * D, 0.0, 2.0);
    uint16_t* k = bf16_array((size_t)T * K * D, 0.0, 2.0);
    uint16_t* wq = bf16_array(D, 0.0, 0.05);
    uint16_t* wk = bf16_array(D, 0.0, 0.05);
    float* cs = malloc(sizeof(float) * MAXPOS * ROT);
    for (int p = 0; p < MAXPOS; ++p)
        for (int i = 0; i < ROT / 2; ++i) {
            double a = p * pow(1.0e4, -2.0 * i / ROT);
            cs[p * ROT + i] = (float)cos(a);
            cs[p * ROT + ROT / 2 + i] = (float)sin(a);
        }
    const int64_t pos[T] = {0, 5, 63, 64, -1, 17};   /* 64 and -1: outside the cache */

    void *dq = to_device(q, sizeof(uint16_t) * T * Q * D);
    void *dk = to_device(k, sizeof(uint16_t) * T * K * D);
    void *dwq = to_device(wq, sizeof(uint16_t) * D), *dwk = to_device(wk, sizeof(uint16_t) * D);
    void *dcs = to_device(cs, sizeof(float) * MAXPOS * ROT), *dpos = to_device(pos, sizeof pos);
    void *dqo = to_device(NULL, sizeof(uint16_t) * T * Q * D);
    void *dko = to_device(NULL, sizeof(uint16_t) * T * K * D);
    mbt_status st = mbt_qknorm_rope(dq, dk, dqo, dko, dwq, dwk, dcs, MAXPOS, dpos, Q, K, T, D,
                                    ROT, eps, delta, MBT_ROPE_ROTATE_HALF, MBT_BF16, NULL);
    check(st == MBT_OK, "mbt_qknorm_rope returned an error");

    uint16_t* gq = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* gk = malloc(sizeof(uint16_t) * T * K * D);
    from_device(gq, dqo, sizeof(uint16_t) * T * Q * D);
    from_device(gk, dko, sizeof(uint16_t) * T * K * D);
    uint16_t* oq = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* ok = malloc(sizeof(uint16_t) * T * K * D);
    check(mbt_ref_qknorm_rope(q, k, oq, ok, wq, wk, cs, MAXPOS, pos, Q, K, T, D, ROT, eps,
                              delta, MBT_REF_ROTATE_HALF, MBT_REF_BF16) == 0,
          "oracle prologue");
    /* the oracle's rounded normalised values, for the rotation allowance */
    uint16_t* nq = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* nk = malloc(sizeof(uint16_t) * T * K * D);
    mbt_ref_rmsnorm_rows(q, nq, wq, (int64_t)T * Q, D, eps, delta, MBT_REF_BF16);
    mbt_ref_rmsnorm_rows(k, nk, wk, (int64_t)T * K, D, eps, delta, MBT_REF_BF16);

    const struct { const uint16_t *g, *o, *n; int heads; const char* name; } sides[2] = {
        {gq, oq, nq, Q, "q"}, {gk, ok, nk, K, "k"}};
    for (int sd = 0; sd < 2; ++sd) {
        long differ = 0, bad = 0;
        for (int t = 0; t < T; ++t) {
            const int inside = pos[t] >= 0 && pos[t] < MAXPOS;
            for (int h = 0; h < sides[sd].heads; ++h)
                for (int c = 0; c < D; ++c) {
                    const size_t e = ((size_t)t * sides[sd].heads + h) * D + c;
                    const int64_t du = ulp_dist(sides[sd].g[e], sides[sd].o[e]);
                    if (du == 0) continue;
                    ++differ;
                    if (du <= 1) continue;
                    if (!inside || c >= ROT) { ++bad; continue; }
                    /* the partner's and the own rounded n may each differ by one
                     * ulp; the rotation moves o by up to (|cos|+|sin|) of that */
                    const int i = c < ROT / 2 ? c : c - ROT / 2;
                    const int pc = c < ROT / 2 ? c + ROT / 2 : c - ROT / 2;
                    const size_t pe = e - c + pc;
                    const double co = fabs(cs[pos[t] * ROT + i]);
                    const double si = fabs(cs[pos[t] * ROT + ROT / 2 + i]);
                    double sp = bf16_spacing(sides[sd].n[e]);
                    if (bf16_spacing(sides[sd].n[pe]) > sp) sp = bf16_spacing(sides[sd].n[pe]);
                    const double bound = (co + si) * sp + bf16_spacing(sides[sd].o[e]);
                    const double diff = fabs((double)mbt_ref_bf16_to_f32(sides[sd].g[e]) -
                                             (double)mbt_ref_bf16_to_f32(sides[sd].o[e]));
                    if (diff > bound) ++bad;
                }
        }
        printf("  %s: %ld of %d elements differ from the oracle, %ld beyond tolerance\n",
               sides[sd].name, differ, T * sides[sd].heads * D, bad);
        check(bad == 0, "prologue beyond tolerance");
        check(differ <= 4 || differ * 200 <= (long)T * sides[sd].heads * D,
              "prologue: too many one-ulp differences");
    }
    hipFree(dq); hipFree(dk); hipFree(dwq); hipFree(dwk); hipFree(dcs); hipFree(dpos);
    hipFree(dqo); hipFree(dko);
    free(q); free(k); free(wq); free(wk); free(cs); free(gq); free(gk); free(oq); free(ok);
    free(nq); free(nk);
}

/* ---- the fused QKV buffer with the key / value cache write -------------- */
static void case_qkv_cache(void) {
    enum { T = 5, Q = 4, K = 2, D = 128, ROT = 64, MAXPOS = 64, NSLOTS = 8 };
    const float eps = 1e-6f;
    printf("case qkv -> q_out + K/V cache: T=%d Q=%d K=%d D=%d, slots of %d\n", T, Q, K, D,
           NSLOTS);
    fflush(stdout);
    const size_t row = (size_t)(Q + 2 * K) * D;               /* elements per token */
    uint16_t* qkv = bf16_array((size_t)T * row, 0.0, 2.0);
    uint16_t* wq = bf16_array(D, 0.0, 0.05);
    uint16_t* wk = bf16_array(D, 0.0, 0.05);
    float* cs = malloc(sizeof(float) * MAXPOS * ROT);
    for (int p = 0; p < MAXPOS; ++p)
        for (int i = 0; i < ROT / 2; ++i) {
            double a = p * pow(1.0e6, -2.0 * i / ROT);
            cs[p * ROT + i] = (float)cos(a);
            cs[p * ROT + ROT / 2 + i] = (float)sin(a);
        }
    const int64_t pos[T] = {3, 9, 70, 12, 40};          /* 70: outside the cache */
    const int64_t slot[T] = {6, 0, 3, -1, 5};           /* -1: padding, no cache row */
    const size_t cache_elems = (size_t)NSLOTS * K * D;
    uint16_t* kc0 = malloc(sizeof(uint16_t) * cache_elems);
    for (size_t e = 0; e < cache_elems; ++e) kc0[e] = 0x7FC0;   /* a NaN fill: rows not written */

    void *dqkv = to_device(qkv, sizeof(uint16_t) * T * row);
    void *dqo = to_device(NULL, sizeof(uint16_t) * T * Q * D);
    void *dkc = to_device(kc0, sizeof(uint16_t) * cache_elems);
    void *dvc = to_device(kc0, sizeof(uint16_t) * cache_elems);
    void *dwq = to_device(wq, sizeof(uint16_t) * D), *dwk = to_device(wk, sizeof(uint16_t) * D);
    void *dcs = to_device(cs, sizeof(float) * MAXPOS * ROT), *dpos = to_device(pos, sizeof pos);
    void *dslot = to_device(slot, sizeof slot);
    mbt_status st = mbt_qkv_norm_rope_cache(dqkv, dqo, dkc, dvc, dslot, NSLOTS, dwq, dwk, dcs,
                                            MAXPOS, dpos, Q, K, T, D, ROT, eps, 1,
                                            MBT_ROPE_ROTATE_HALF, MBT_BF16, 0, NULL);
    check(st == MBT_OK, "mbt_qkv_norm_rope_cache returned an error");
    uint16_t* gq = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* gkc = malloc(sizeof(uint16_t) * cache_elems);
    uint16_t* gvc = malloc(sizeof(uint16_t) * cache_elems);
    from_device(gq, dqo, sizeof(uint16_t) * T * Q * D);
    from_device(gkc, dkc, sizeof(uint16_t) * cache_elems);
    from_device(gvc, dvc, sizeof(uint16_t) * cache_elems);

    /* the oracle's prologue on the q and k heads gathered out of qkv */
    uint16_t* q = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* k = malloc(sizeof(uint16_t) * T * K * D);
    for (int t = 0; t < T; ++t) {
        memcpy(q + (size_t)t * Q * D, qkv + t * row, sizeof(uint16_t) * Q * D);
        memcpy(k + (size_t)t * K * D, qkv + t * row + (size_t)Q * D, sizeof(uint16_t) * K * D);
    }
    uint16_t* oq = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* ok = malloc(sizeof(uint16_t) * T * K * D);
    check(mbt_ref_qknorm_rope(q, k, oq, ok, wq, wk, cs, MAXPOS, pos, Q, K, T, D, ROT, eps, 1,
                              MBT_REF_ROTATE_HALF, MBT_REF_BF16) == 0, "oracle prologue");
    long far = 0, differ = 0, vbad = 0, untouched_bad = 0;
    for (size_t e = 0; e < (size_t)T * Q * D; ++e) {
        const int64_t d = ulp_dist(gq[e], oq[e]);
        differ += d != 0;
        far += d > 1;
    }
    int written[NSLOTS] = {0};
    for (int t = 0; t < T; ++t) {
        if (slot[t] < 0 || slot[t] >= NSLOTS) continue;
        written[slot[t]] = 1;
        for (size_t e = 0; e < (size_t)K * D; ++e) {
            const size_t c = (size_t)slot[t] * K * D + e;
            const int64_t d = ulp_dist(gkc[c], ok[(size_t)t * K * D + e]);
            differ += d != 0;
            far += d > 1;
            vbad += gvc[c] != qkv[t * row + (size_t)(Q + K) * D + e];
        }
    }
    for (int sl = 0; sl < NSLOTS; ++sl)
        if (!written[sl])
            for (size_t e = 0; e < (size_t)K * D; ++e)
                untouched_bad += gkc[(size_t)sl * K * D + e] != 0x7FC0 ||
                                 gvc[(size_t)sl * K * D + e] != 0x7FC0;
    printf("  q and cached keys: %ld differ, %ld by more than one ulp; value rows not copied "
           "bit for bit: %ld; unwritten cache elements changed: %ld\n", differ, far, vbad,
           untouched_bad);
    check(far == 0, "qkv cache: beyond one ulp");
    check(vbad == 0, "value rows not copied bit for bit");
    check(untouched_bad == 0, "a cache row without a token was written");
    hipFree(dqkv); hipFree(dqo); hipFree(dkc); hipFree(dvc); hipFree(dwq); hipFree(dwk);
    hipFree(dcs); hipFree(dpos); hipFree(dslot);
    free(qkv); free(wq); free(wk); free(cs); free(kc0); free(gq); free(gkc); free(gvc);
    free(q); free(k); free(oq); free(ok);
}

/* ---- residual-add RMSNorm to FP8 ---------------------------------------- */
static void case_norm_fp8(void) {
    enum { T = 7, H = 1024 };
    const float eps = 1e-6f;
    printf("case residual RMSNorm -> FP8: T=%d H=%d bf16\n", T, H);
    fflush(stdout);
    uint16_t* x = bf16_array((size_t)T * H, 0.0, 1.0);
    uint16_t* r = bf16_array((size_t)T * H, 0.0, 1.0);
    uint16_t* w = bf16_array(H, 1.0, 0.05);
    /* the static scale from the oracle's calibration pass on these rows */
    const float amax = mbt_ref_fused_add_rmsnorm_amax(x, r, w, T, H, eps, 0, MBT_REF_BF16);
    const float inv_scale = (float)(448.0 / (double)amax);
    void *dx = to_device(x, sizeof(uint16_t) * T * H), *dr = to_device(r, sizeof(uint16_t) * T * H);
    void *dw = to_device(w, sizeof(uint16_t) * H), *dy = to_device(NULL, (size_t)T * H);
    mbt_status st = mbt_fused_add_rmsnorm_fp8(dx, dr, dw, dy, inv_scale, T, H, eps, 0, MBT_BF16,
                                              NULL);
    check(st == MBT_OK, "mbt_fused_add_rmsnorm_fp8 returned an error");
    uint8_t* gy = malloc((size_t)T * H);
    uint16_t* gr = malloc(sizeof(uint16_t) * T * H);
    from_device(gy, dy, (size_t)T * H);
    from_device(gr, dr, sizeof(uint16_t) * T * H);
    uint8_t* oy = malloc((size_t)T * H);
    check(mbt_ref_fused_add_rmsnorm_fp8(x, r, w, oy, inv_scale, T, H, eps, 0, MBT_REF_BF16) == 0,
          "oracle norm fp8");                   /* updates r in place: the oracle's residual */
    long differ = 0, far = 0, res_bad = 0;
    for (size_t e = 0; e < (size_t)T * H; ++e) {
        const int a = (gy[e] & 0x80) ? -(gy[e] & 0x7F) : (gy[e] & 0x7F);
        const int b = (oy[e] & 0x80) ? -(oy[e] & 0x7F) : (oy[e] & 0x7F);
        const int d = abs(a - b);
        if (d) ++differ;
        if (d > 1) ++far;
        if (gr[e] != r[e]) ++res_bad;
    }
    printf("  FP8 codes: %ld of %d differ (all by one step: %s); residual: %ld not bit-identical\n",
           differ, T * H, far ? "no" : "yes", res_bad);
    check(far == 0, "FP8 codes more than one step apart");
    check(differ <= 4 || differ * 500 <= (long)T * H, "FP8: too many one-step differences");
    check(res_bad == 0, "residual sum not bit-identical");
    hipFree(dx); hipFree(dr); hipFree(dw); hipFree(dy);
    free(x); free(r); free(w); free(gy); free(gr); free(oy);
}

/* ---- gated SiLU --------------------------------------------------------- */
static void case_gated_act(void) {
    enum { T = 3, DH = 1024 };
    printf("case gated SiLU: T=%d d=%d bf16\n", T, DH);
    fflush(stdout);
    uint16_t* gu = bf16_array((size_t)T * 2 * DH, 0.0, 1.5);
    void *dgu = to_device(gu, sizeof(uint16_t) * T * 2 * DH);
    void *dout = to_device(NULL, sizeof(uint16_t) * T * DH);
    mbt_status st = mbt_gated_act(dgu, dout, T, DH, MBT_ACT_SILU, MBT_BF16, NULL);
    check(st == MBT_OK, "mbt_gated_act returned an error");
    uint16_t* g = malloc(sizeof(uint16_t) * T * DH);
    uint16_t* o = malloc(sizeof(uint16_t) * T * DH);
    from_device(g, dout, sizeof(uint16_t) * T * DH);
    check(mbt_ref_gated_act(gu, o, T, DH, MBT_REF_SILU, MBT_REF_BF16) == 0, "oracle act");
    long differ = 0, far = 0;
    for (size_t e = 0; e < (size_t)T * DH; ++e) {
        const int64_t d = ulp_dist(g[e], o[e]);
        if (d) ++differ;
        if (d > 1) ++far;
    }
    printf("  %ld of %d differ from the oracle, %ld by more than one ulp\n", differ, T * DH, far);
    check(far == 0, "activation beyond one ulp");
    check(differ <= 4 || differ * 200 <= (long)T * DH, "activation: too many differences");
    hipFree(dgu); hipFree(dout);
    free(gu); free(g); free(o);
}

/* ---- the adaptive norm to FP8, with its calibration pass ---------------- */
static void case_adarms_fp8(void) {
    enum { T = 4, H = 512 };
    const float eps = 1e-6f;
    printf("case adaptive RMSNorm -> FP8: T=%d H=%d bf16, gated residual, calibrated\n", T, H);
    fflush(stdout);
    uint16_t* x = bf16_array((size_t)T * H, 0.0, 1.0);
    uint16_t* r = bf16_array((size_t)T * H, 0.0, 1.0);
    uint16_t* gate = bf16_array(H, 1.0, 0.1);
    uint16_t* scale = bf16_array(H, 0.0, 0.1);
    uint16_t* shift = bf16_array(H, 0.0, 0.1);
    void *dx = to_device(x, sizeof(uint16_t) * T * H), *dr = to_device(r, sizeof(uint16_t) * T * H);
    void *dg = to_device(gate, sizeof(uint16_t) * H), *dsc = to_device(scale, sizeof(uint16_t) * H);
    void *dsh = to_device(shift, sizeof(uint16_t) * H), *dy = to_device(NULL, (size_t)T * H);
    const float zero = 0.0f;
    void* damax = to_device(&zero, sizeof zero);      /* the caller zeroes the fold */
    /* calibration on the GPU and in the oracle: the same maximum */
    mbt_status st = mbt_adarms_amax(dx, dr, dg, dsc, dsh, (float*)damax, T, H, eps, MBT_BF16,
                                    NULL);
    check(st == MBT_OK, "mbt_adarms_amax returned an error");
    float gamax = 0.0f;
    from_device(&gamax, damax, sizeof gamax);
    const float amax = mbt_ref_adarms_amax(x, r, gate, scale, shift, T, H, eps, MBT_REF_BF16);
    check(fabs((double)gamax - (double)amax) <= 1e-5 * (double)amax, "calibration amax");
    const float inv_scale = (float)(448.0 / (double)amax);
    st = mbt_adarms_fp8(dx, dr, dg, dsc, dsh, (uint8_t*)dy, inv_scale, T, H, eps, MBT_BF16, NULL);
    check(st == MBT_OK, "mbt_adarms_fp8 returned an error");
    uint8_t* gy = malloc((size_t)T * H);
    uint16_t* gr = malloc(sizeof(uint16_t) * T * H);
    from_device(gy, dy, (size_t)T * H);
    from_device(gr, dr, sizeof(uint16_t) * T * H);
    uint8_t* oy = malloc((size_t)T * H);
    check(mbt_ref_adarms_fp8(x, r, gate, scale, shift, oy, inv_scale, T, H, eps,
                             MBT_REF_BF16) == 0, "oracle adaptive norm fp8");
    long differ = 0, far = 0, res_bad = 0;
    for (size_t e = 0; e < (size_t)T * H; ++e) {
        const int a = (gy[e] & 0x80) ? -(gy[e] & 0x7F) : (gy[e] & 0x7F);
        const int b = (oy[e] & 0x80) ? -(oy[e] & 0x7F) : (oy[e] & 0x7F);
        const int d = abs(a - b);
        if (d) ++differ;
        if (d > 1) ++far;
        if (gr[e] != r[e]) ++res_bad;
    }
    printf("  amax %.9g vs %.9g; FP8 codes: %ld of %d differ, %ld by more than one step; "
           "residual: %ld not bit-identical\n", gamax, amax, differ, T * H, far, res_bad);
    check(far == 0, "adaptive FP8 codes more than one step apart");
    check(differ <= 4 || differ * 500 <= (long)T * H, "adaptive FP8: too many differences");
    check(res_bad == 0, "gated residual sum not bit-identical");
    hipFree(dx); hipFree(dr); hipFree(dg); hipFree(dsc); hipFree(dsh); hipFree(dy);
    hipFree(damax);
    free(x); free(r); free(gate); free(scale); free(shift); free(gy); free(gr); free(oy);
}

/* ---- the standalone rotation (the split route), interleaved pairs ------- */
static void case_rope(void) {
    enum { T = 5, Q = 3, K = 1, D = 64, ROT = 32, MAXPOS = 40 };
    printf("case rope: T=%d Q=%d K=%d D=%d rot=%d bf16, interleaved, in place\n", T, Q, K, D,
           ROT);
    fflush(stdout);
    uint16_t* q = bf16_array((size_t)T * Q * D, 0.0, 1.0);
    uint16_t* k = bf16_array((size_t)T * K * D, 0.0, 1.0);
    float* cs = malloc(sizeof(float) * MAXPOS * ROT);
    for (int p = 0; p < MAXPOS; ++p)
        for (int i = 0; i < ROT / 2; ++i) {
            double a = p * pow(1.0e4, -2.0 * i / ROT);
            cs[p * ROT + i] = (float)cos(a);
            cs[p * ROT + ROT / 2 + i] = (float)sin(a);
        }
    const int64_t pos[T] = {3, 39, 40, -2, 0};      /* 40 and -2: untouched */
    void *dq = to_device(q, sizeof(uint16_t) * T * Q * D);
    void *dk = to_device(k, sizeof(uint16_t) * T * K * D);
    void *dcs = to_device(cs, sizeof(float) * MAXPOS * ROT), *dpos = to_device(pos, sizeof pos);
    mbt_status st = mbt_rope(dq, dk, dcs, MAXPOS, dpos, Q, K, T, D, ROT, MBT_ROPE_INTERLEAVED,
                             MBT_BF16, NULL);
    check(st == MBT_OK, "mbt_rope returned an error");
    uint16_t* gq = malloc(sizeof(uint16_t) * T * Q * D);
    uint16_t* gk = malloc(sizeof(uint16_t) * T * K * D);
    from_device(gq, dq, sizeof(uint16_t) * T * Q * D);
    from_device(gk, dk, sizeof(uint16_t) * T * K * D);
    check(mbt_ref_rope(q, cs, MAXPOS, pos, T, Q, D, ROT, MBT_REF_INTERLEAVED, MBT_REF_BF16) == 0,
          "oracle rope q");
    check(mbt_ref_rope(k, cs, MAXPOS, pos, T, K, D, ROT, MBT_REF_INTERLEAVED, MBT_REF_BF16) == 0,
          "oracle rope k");
    long differ = 0;
    for (size_t e = 0; e < (size_t)T * Q * D; ++e) differ += gq[e] != q[e];
    for (size_t e = 0; e < (size_t)T * K * D; ++e) differ += gk[e] != k[e];
    printf("  %ld elements differ from the oracle (the rotation is bit-exact)\n", differ);
    check(differ == 0, "standalone rotation not bit-identical to the oracle");
    hipFree(dq); hipFree(dk); hipFree(dcs); hipFree(dpos);
    free(q); free(k); free(cs); free(gq); free(gk);
}

/* ---- a rejected call: nothing launched, a status and a detail string --- */
static void case_rejected(void) {
    printf("case rejected call: an unknown dtype\n");
    fflush(stdout);
    mbt_status st = mbt_gated_act((const void*)16, (void*)16, 1, 8, MBT_ACT_SILU, 99, NULL);
    check(st == MBT_ERR_BAD_DTYPE, "unknown dtype not refused");
    check(strlen(mbt_last_error()) > 0, "no detail string for a refused call");
    check(strcmp(mbt_status_string(st), "MBT_ERR_BAD_DTYPE") == 0, "status name");
    check(mbt_abi_version() == MBT_ABI_VERSION, "ABI version");
}

int main(void) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    case_rejected();
    case_prologue();
    case_qkv_cache();
    case_norm_fp8();
    case_gated_act();
    case_rope();
    case_adarms_fp8();
    printf(failures ? "c abi: %d failure(s)\n" : "c abi: every check passed\n", failures);
    return failures ? 1 : 0;
}
