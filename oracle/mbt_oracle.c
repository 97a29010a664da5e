/*
 * mbt_oracle.c -- plain, single-threaded CPU oracle (TEST INFRASTRUCTURE).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use
 * this file.  It shares no code with the HIP path.  Build:
 *   gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -lm
 * (oracle/build.py does exactly that).
 *
 * Sources followed, by page and section:
 *  [P1] "thox-edge-ops v2: fused decode kernels for small models on THOX edge
 *       hardware": section 3 (requirements R1 numerics, R2 conventions, R5
 *       safety), section 5.1 (the six operators; the display formulas did
 *       not survive, only the prose that frames them), section 5.4 (fused
 *       QK-norm and RoPE), section 7.5 (numerics contract).
 *  [P2] ninfer PR #273, "Register the text profile of ops::rmsnorm_rope ...",
 *       section "Implementation" (rotation consumes the rounded normalised
 *       value; weight as a delta around one; out of place).
 *  [P3] FlashRT "optimization details" (Pi0.5 on Jetson AGX Thor): fused
 *       kernel table and the static FP8 calibration paragraph.
 *  GELU-tanh constants: Hendrycks and Gimpel, "Gaussian Error Linear Units"
 *  (reference [9] of P1).  RMSNorm: Zhang and Sennrich (reference [5] of P1).
 *
 * Readings taken where the pages are silent are listed in the design notes;
 * the ones that shape arithmetic are repeated next to the code below.
 *
 * The MBT_ORACLE_MUTATION switch plants one deliberate mistake per value.  It
 * is off (0) in every build that tests, smoke or bench use; the tests build
 * mutated copies only to prove that the pins would catch such a mistake.
 */
#include "mbt_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifndef MBT_ORACLE_MUTATION
#define MBT_ORACLE_MUTATION 0
#endif

/* ------------------------------------------------------------------------ */
/* Converters, written from the IEEE 754 binary16 / bfloat16 definitions and */
/* the OCP 8-bit floating point (OFP8) E4M3 definition.                      */
/* ------------------------------------------------------------------------ */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 is the upper half of a binary32: decoding is exact. */
float mbt_ref_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even.  NaN stays a quiet
 * NaN with its sign; overflow rounds to infinity. */
uint16_t mbt_ref_f32_to_bf16(float f) {
    uint32_t u = f2u(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
#if MBT_ORACLE_MUTATION == 9
    return (uint16_t)(u >> 16);                       /* planted: truncation */
#else
    uint32_t keep = u >> 16, rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
#endif
}

/* binary16 -> binary32: exact, including subnormals. */
float mbt_ref_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0x1fu)                                   /* inf / NaN */
        return u2f(sign | 0x7f800000u | (m << 13));
    if (e == 0) {                                     /* zero / subnormal */
        float v = ldexpf((float)m, -24);              /* m * 2^-24, exact */
        return sign ? -v : v;
    }
    return u2f(sign | ((e + 112u) << 23) | (m << 13));
}

/* binary32 -> binary16, round to nearest, ties to even; subnormal results
 * are produced, magnitudes that round past 65504 become infinity. */
uint16_t mbt_ref_f32_to_f16(float f) {
    uint32_t u = f2u(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
    if (a == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);
    int32_t e = (int32_t)(a >> 23) - 127;             /* unbiased exponent */
    uint32_t m = a & 0x7fffffu;
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    if (e >= -14) {                                   /* normal binary16 */
        uint32_t half = ((uint32_t)(e + 15) << 10) | (m >> 13);
        uint32_t rest = m & 0x1fffu;
#if MBT_ORACLE_MUTATION == 24
        (void)rest;                                   /* planted: truncation */
#else
        if (rest > 0x1000u || (rest == 0x1000u && (half & 1u))) half += 1u;
#endif
        return (uint16_t)(sign | half);               /* a carry may reach inf */
    }
    if (e < -25) return sign;                         /* below half the least subnormal */
    /* value = (2^23 + m) * 2^(e-23); in units of 2^-24 that is
     * (2^23 + m) * 2^(e+1): drop -(e+1) bits with round to nearest even. */
    uint32_t full = m | 0x800000u;
    int shift = -(e + 1);                             /* 14 .. 24 */
    uint32_t q = full >> shift;
    uint32_t rest = full & ((1u << shift) - 1u);
    uint32_t halfway = 1u << (shift - 1);
    if (rest > halfway || (rest == halfway && (q & 1u))) q += 1u;
    return (uint16_t)(sign | q);                      /* q == 0x400 is the least normal */
}

/* OCP E4M3 ("fn": no infinities, one NaN pattern per sign, max 448):
 * exponent bias 7, 3 mantissa bits, subnormals m/8 * 2^-6. */
float mbt_ref_e4m3fn_to_f32(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    float v;
    if (e == 0xf && m == 7) return s ? -NAN : NAN;
    if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -v : v;
}

/* binary32 -> E4M3 with saturation: NaN -> 0x7f (sign kept), |v| > 448 ->
 * +-448, otherwise round to nearest, ties to even (the quantization the
 * FP8 variants apply; saturation is the reading taken for out-of-range
 * values, since a static scale calibrated on other data can overshoot). */
uint8_t mbt_ref_f32_to_e4m3fn(float f) {
    uint8_t sign = (f2u(f) >> 24) & 0x80u;
    if (isnan(f)) return (uint8_t)(sign | 0x7fu);
    float a = fabsf(f);
#if MBT_ORACLE_MUTATION == 29
    if (a > 448.0f) return (uint8_t)(sign | 0x7fu);  /* planted: overflow to NaN */
#else
    if (a > 448.0f) return (uint8_t)(sign | 0x7eu);
#endif
    if (a < 0.015625f) {                              /* below 2^-6: subnormal grid 2^-9 */
#if MBT_ORACLE_MUTATION == 8
        float q = truncf(ldexpf(a, 9));               /* planted: truncation */
#else
        float q = rintf(ldexpf(a, 9));                /* exact scaling, RNE */
#endif
        return (uint8_t)(sign | (uint8_t)q);          /* q == 8 is the least normal */
    }
    int ex;
    float fr = frexpf(a, &ex);                        /* a = fr * 2^ex, fr in [0.5,1) */
    int e = ex - 1;                                   /* a = (2 fr) * 2^e, e in [-6, 8] */
#if MBT_ORACLE_MUTATION == 8
    float q = truncf((2.0f * fr - 1.0f) * 8.0f);
#else
    float q = rintf((2.0f * fr - 1.0f) * 8.0f);       /* exact operands, RNE */
#endif
    int qi = (int)q;
    if (qi == 8) { qi = 0; e += 1; }
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | qi));
}

/* ---- element access by dtype -------------------------------------------- */

static float ld(const void* p, int64_t i, int32_t dtype) {
    switch (dtype) {
    case MBT_REF_F32: return ((const float*)p)[i];
    case MBT_REF_F16: return mbt_ref_f16_to_f32(((const uint16_t*)p)[i]);
    default:          return mbt_ref_bf16_to_f32(((const uint16_t*)p)[i]);
    }
}

/* R(v): the single rounding of an output to its dtype. */
static void st(void* p, int64_t i, int32_t dtype, float v) {
    switch (dtype) {
    case MBT_REF_F32: ((float*)p)[i] = v; break;
    case MBT_REF_F16: ((uint16_t*)p)[i] = mbt_ref_f32_to_f16(v); break;
    default:          ((uint16_t*)p)[i] = mbt_ref_f32_to_bf16(v); break;
    }
}

/* R(v) read back as fp32 (the value a later step of a fused op consumes). */
static float rounded(float v, int32_t dtype) {
    switch (dtype) {
    case MBT_REF_F32: return v;
    case MBT_REF_F16: return mbt_ref_f16_to_f32(mbt_ref_f32_to_f16(v));
    default:          return mbt_ref_bf16_to_f32(mbt_ref_f32_to_bf16(v));
    }
}

static int dtype_ok(int32_t dtype) {
    return dtype == MBT_REF_F32 || dtype == MBT_REF_F16 || dtype == MBT_REF_BF16;
}

void mbt_ref_encode(const float* in, void* out, int64_t n, int32_t dtype) {
    for (int64_t i = 0; i < n; i++) st(out, i, dtype, in[i]);
}
void mbt_ref_decode(const void* in, float* out, int64_t n, int32_t dtype) {
    for (int64_t i = 0; i < n; i++) out[i] = ld(in, i, dtype);
}
void mbt_ref_encode_e4m3fn(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = mbt_ref_f32_to_e4m3fn(in[i]);
}
void mbt_ref_decode_e4m3fn(const uint8_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = mbt_ref_e4m3fn_to_f32(in[i]);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm (P1 5.1; weight convention of P1 section 2: Llama multiplies by w, */
/* Gemma by 1 + w formed in fp32; delta selects between them).               */
/* ------------------------------------------------------------------------ */

/* inv = 1 / sqrt(mean over all D channels of x^2 + eps), accumulated in
 * fp32 in index order.  `x` holds D values already decoded to fp32. */
static float inv_rms(const float* x, int32_t D, int32_t rot_dim, float eps) {
    float ss = 0.0f;
    for (int32_t i = 0; i < D; i++) ss += x[i] * x[i];
    (void)rot_dim;
#if MBT_ORACLE_MUTATION == 2
    eps = 0.0f;                                       /* planted: eps dropped */
#endif
#if MBT_ORACLE_MUTATION == 3
    if (rot_dim > 0) return 1.0f / sqrtf(ss / (float)rot_dim + eps); /* planted */
#endif
#if MBT_ORACLE_MUTATION == 28
    if (D > 1) return 1.0f / sqrtf(ss / (float)(D - 1) + eps); /* planted: D - 1 */
#endif
#if MBT_ORACLE_MUTATION == 33
    return 1.0f / (sqrtf(ss / (float)D) + eps);       /* planted: eps outside the root */
#endif
    return 1.0f / sqrtf(ss / (float)D + eps);
}

static float weight_term(const void* w, int64_t i, int32_t dtype, int32_t delta) {
#if MBT_ORACLE_MUTATION == 6
    (void)delta; return ld(w, i, dtype);              /* planted: offset ignored */
#else
    return ld(w, i, dtype) + (float)delta;
#endif
}

/* (x * inv) times the weight term; with no weight (w == NULL, the norm's
 * scale folded into the next GEMM's weights: FlashRT optimization details,
 * the weight-folding paragraph) the product is used as it is. */
static float apply_weight(float xn, const void* w, int64_t i, int32_t dtype, int32_t delta) {
#if MBT_ORACLE_MUTATION == 36
    xn = rounded(xn, dtype);                 /* planted: x * inv rounded before the weight */
#endif
    if (w) return xn * weight_term(w, i, dtype, delta);
#if MBT_ORACLE_MUTATION == 13
    return xn * 2.0f;                    /* planted: a missing weight read as 1 + 1 */
#else
    return xn;
#endif
}

/* The value an FP8 epilogue (or its calibration pass) consumes: the fp32
 * result itself, quantized once (FlashRT optimization details, static FP8:
 * the fused kernels go from the fp32 value straight to the 8-bit code), never
 * its copy already rounded to the I/O dtype.  `site` names the epilogue for
 * the planted-mistake switch. */
static float fp8_source(float v, int32_t dtype, int site) {
#if MBT_ORACLE_MUTATION >= 17 && MBT_ORACLE_MUTATION <= 22
    if (site == MBT_ORACLE_MUTATION) return rounded(v, dtype); /* planted: double rounding */
#endif
    (void)dtype; (void)site;
    return v;
}

/* |v|: a calibration pass takes the largest magnitude. */
static float magnitude(float v) {
#if MBT_ORACLE_MUTATION == 30
    return v;                                         /* planted: signed maximum */
#else
    return fabsf(v);
#endif
}

int mbt_ref_rmsnorm_rows(const void* x, void* y, const void* w, int64_t rows,
                         int32_t D, float eps, int32_t weight_offset,
                         int32_t dtype) {
    if (!dtype_ok(dtype) || D <= 0 || rows < 0 || (weight_offset & ~1) ||
        (!w && weight_offset))
        return -1;
    float xs[4096];
    if (D > 4096) return -1;
    for (int64_t r = 0; r < rows; r++) {
        for (int32_t i = 0; i < D; i++) xs[i] = ld(x, r * D + i, dtype);
        float inv = inv_rms(xs, D, 0, eps);
        for (int32_t i = 0; i < D; i++)
            st(y, r * D + i, dtype, apply_weight(xs[i] * inv, w, i, dtype, weight_offset));
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Rotary embedding (P1 5.1): pairs (a_i, b_i) = (i, i + rot/2) for the       */
/* rotate-half layout, (2i, 2i+1) for the interleaved one, i < rot/2, with    */
/* c = cos, s = sin of the cached angle of the token's position:              */
/*   o_a = a c - b s,  o_b = b c + a s  (each product rounded on its own).    */
/* ------------------------------------------------------------------------ */

static void pair_index(int32_t i, int32_t rot, int32_t layout, int32_t* a, int32_t* b) {
    if (layout == MBT_REF_ROTATE_HALF) {
#if MBT_ORACLE_MUTATION == 5
        *a = i; *b = (i + rot / 2 + 1) % rot;         /* planted: partner off by one */
#else
        *a = i; *b = i + rot / 2;
#endif
    } else {
        *a = 2 * i; *b = 2 * i + 1;
    }
}

/* Position range check (P1 R5 and 5.4): only 0 <= p < max_pos reads the
 * cache; any other position has no cache row and the result is NULL. */
static const float* cache_row(const float* cos_sin, int64_t p, int64_t max_pos,
                              int32_t rot) {
#if MBT_ORACLE_MUTATION == 12
    if (p >= max_pos && max_pos > 0) p = max_pos - 1; /* planted: clamp */
#endif
#if MBT_ORACLE_MUTATION == 26
    if (p >= max_pos - 1) return NULL;                /* planted: last row outside */
#endif
#if MBT_ORACLE_MUTATION == 32
    if (p < 0 && p >= -max_pos) p += max_pos;         /* planted: negative wraps */
#endif
    if (p < 0 || p >= max_pos) return NULL;
    return cos_sin + p * (int64_t)rot;
}

/* Rotate one head's first rot channels: `n` holds D fp32 values (already
 * rounded to the dtype), `o` receives D fp32 values before output rounding. */
static void rotate_head(const float* n, float* o, int32_t D, int32_t rot,
                        int32_t layout, const float* cs) {
    for (int32_t i = 0; i < D; i++) o[i] = n[i];
    for (int32_t i = 0; i < rot / 2; i++) {
        int32_t a, b;
        pair_index(i, rot, layout, &a, &b);
        float c = cs[i], s = cs[rot / 2 + i];
#if MBT_ORACLE_MUTATION == 25
        if (layout == MBT_REF_INTERLEAVED) {          /* planted: channel index */
            c = cs[(2 * i) % (rot / 2)];
            s = cs[rot / 2 + (2 * i) % (rot / 2)];
        }
#endif
#if MBT_ORACLE_MUTATION == 4
        s = -s;                                        /* planted: wrong sign */
#endif
        float oa = n[a] * c - n[b] * s;
#if MBT_ORACLE_MUTATION == 31
        float ob = n[b] * c - n[a] * s;                /* planted: o_b sign */
#else
        float ob = n[b] * c + n[a] * s;
#endif
#if MBT_ORACLE_MUTATION == 1
        oa *= 1.000001f; ob *= 1.000001f;              /* planted: strength control */
#endif
        o[a] = oa;
        o[b] = ob;
    }
}

static int rope_args_ok(int32_t D, int32_t rot, int32_t layout, int32_t dtype) {
    return dtype_ok(dtype) && D > 0 && D <= 4096 && rot >= 0 && rot <= D &&
           (rot % 2) == 0 &&
           (layout == MBT_REF_ROTATE_HALF || layout == MBT_REF_INTERLEAVED);
}

int mbt_ref_rope(void* x, const float* cos_sin, int64_t max_pos,
                 const int64_t* pos, int64_t T, int32_t heads, int32_t D,
                 int32_t rot_dim, int32_t layout, int32_t dtype) {
    if (!rope_args_ok(D, rot_dim, layout, dtype) || heads < 0 || T < 0) return -1;
    float n[4096], o[4096];
    for (int64_t t = 0; t < T; t++) {
        const float* cs = cache_row(cos_sin, pos[t], max_pos, rot_dim);
        if (!cs) continue;                            /* untouched */
        for (int32_t h = 0; h < heads; h++) {
            int64_t base = (t * heads + h) * (int64_t)D;
            for (int32_t i = 0; i < D; i++) n[i] = ld(x, base + i, dtype);
            rotate_head(n, o, D, rot_dim, layout, cs);
            for (int32_t i = 0; i < rot_dim; i++) st(x, base + i, dtype, o[i]);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Fused QK-norm + RoPE (P1 5.1 and 5.4; P2 "Implementation"): for every     */
/* token, each of its Q query heads is normalised with w_q and each of its K */
/* key heads with w_k (weights of length head_dim), the normalised value is  */
/* rounded to the I/O dtype, and that rounded value is rotated.  A token     */
/* positioned beyond the cache gets the norm only; its rotation is skipped.   */
/* Written out on its own (not by calling the two primitives above) so the   */
/* tests can check that this op equals their composition.                    */
/* ------------------------------------------------------------------------ */

/* round_first = 1: the normalised value is rounded to the dtype and that
 * rounded value is rotated (the contract of the fused op, P1 5.1 and P2
 * "Implementation").  round_first = 0: the single-rounding variant the P2
 * review asks for (review item 1): the rotated channels take the fp32 norm
 * result straight into the rotation and are rounded once, after it; the
 * channels past rot_dim (and every channel of a token outside the cache)
 * are the norm result rounded once, as in the contract. */
static void norm_rope_head(const void* in, void* out, int64_t base,
                           const void* w, int32_t D, int32_t rot,
                           float eps, int32_t delta, int32_t layout,
                           int32_t dtype, const float* cs /* NULL: no rotation */,
                           int round_first) {
    float x[4096], n[4096], o[4096];
    for (int32_t i = 0; i < D; i++) x[i] = ld(in, base + i, dtype);
    float inv = inv_rms(x, D, rot, eps);
    for (int32_t i = 0; i < D; i++) {
        n[i] = (x[i] * inv) * weight_term(w, i, dtype, delta);
#if MBT_ORACLE_MUTATION == 14
        round_first = 1;                          /* planted: single rounding ignored */
#endif
        if (round_first) n[i] = rounded(n[i], dtype);
    }
    if (cs) rotate_head(n, o, D, rot, layout, cs);
    else for (int32_t i = 0; i < D; i++) o[i] = n[i];
    for (int32_t i = 0; i < D; i++) st(out, base + i, dtype, o[i]);
}

static int qknorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                       const void* w_q, const void* w_k, const float* cos_sin,
                       int64_t max_pos, const int64_t* pos, int32_t Q, int32_t K,
                       int64_t T, int32_t head_dim, int32_t rot_dim, float eps,
                       int32_t weight_offset, int32_t layout, int32_t dtype,
                       int round_first) {
    if (!rope_args_ok(head_dim, rot_dim, layout, dtype) || Q < 0 || K < 0 ||
        T < 0 || (weight_offset & ~1) || max_pos < 0)
        return -1;
    const int32_t D = head_dim;
    for (int64_t t = 0; t < T; t++) {
        const float* cs = cache_row(cos_sin, pos[t], max_pos, rot_dim);
        for (int32_t h = 0; h < Q; h++)
            norm_rope_head(q_in, q_out, (t * Q + h) * (int64_t)D, w_q, D, rot_dim,
                           eps, weight_offset, layout, dtype, cs, round_first);
        for (int32_t h = 0; h < K; h++)
#if MBT_ORACLE_MUTATION == 11
            (void)w_k,
            norm_rope_head(k_in, k_out, (t * K + h) * (int64_t)D, w_q, D, rot_dim,
                           eps, weight_offset, layout, dtype, cs, round_first); /* planted */
#else
            norm_rope_head(k_in, k_out, (t * K + h) * (int64_t)D, w_k, D, rot_dim,
                           eps, weight_offset, layout, dtype, cs, round_first);
#endif
    }
    return 0;
}

int mbt_ref_qknorm_rope(const void* q_in, const void* k_in, void* q_out,
                        void* k_out, const void* w_q, const void* w_k,
                        const float* cos_sin, int64_t max_pos,
                        const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                        int32_t head_dim, int32_t rot_dim, float eps,
                        int32_t weight_offset, int32_t layout, int32_t dtype) {
    return qknorm_rope(q_in, k_in, q_out, k_out, w_q, w_k, cos_sin, max_pos, pos, Q, K, T,
                       head_dim, rot_dim, eps, weight_offset, layout, dtype, 1);
}

int mbt_ref_qknorm_rope_round_once(const void* q_in, const void* k_in, void* q_out,
                                   void* k_out, const void* w_q, const void* w_k,
                                   const float* cos_sin, int64_t max_pos,
                                   const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                                   int32_t head_dim, int32_t rot_dim, float eps,
                                   int32_t weight_offset, int32_t layout, int32_t dtype) {
    return qknorm_rope(q_in, k_in, q_out, k_out, w_q, w_k, cos_sin, max_pos, pos, Q, K, T,
                       head_dim, rot_dim, eps, weight_offset, layout, dtype, 0);
}

/* ------------------------------------------------------------------------ */
/* Fused residual-add RMSNorm (P1 5.1: the sum is written back to the        */
/* residual stream and its rounded value is what gets normalised; R1: that   */
/* sum matches eager addition bit for bit, i.e. it is the fp32 add of the    */
/* decoded operands rounded once to the dtype).                              */
/* ------------------------------------------------------------------------ */

/* s[i] (fp32 value of the rounded sum) for row t; writes the residual when
 * `write_res`.  Returns nothing; `s` receives H values. */
static void residual_sum(const void* x, void* residual, int64_t t, int32_t H,
                         int32_t dtype, int write_res, float* s) {
    for (int32_t i = 0; i < H; i++) {
        int64_t k = t * H + i;
        float xv = ld(x, k, dtype);
        if (residual) {
            float sum = xv + ld(residual, k, dtype);
#if MBT_ORACLE_MUTATION == 10
            s[i] = sum;                               /* planted: sum not rounded */
#else
            s[i] = rounded(sum, dtype);
#endif
#if MBT_ORACLE_MUTATION == 34
            (void)write_res;                          /* planted: residual not updated */
#else
            if (write_res) st(residual, k, dtype, sum);
#endif
        } else {
            s[i] = xv;
        }
    }
}

/* A missing weight (w == NULL) admits no offset: there is nothing to add it to. */
static int norm_args_ok(const void* w, int64_t T, int32_t H, int32_t delta, int32_t dtype) {
    return dtype_ok(dtype) && T >= 0 && H > 0 && !(delta & ~1) && (w || delta == 0);
}

int mbt_ref_fused_add_rmsnorm(void* x, void* residual, const void* w,
                              int64_t T, int32_t H, float eps,
                              int32_t weight_offset, int32_t dtype) {
    if (!norm_args_ok(w, T, H, weight_offset, dtype)) return -1;
    float* s = (float*)malloc((size_t)H * sizeof(float));
    if (!s) return -1;
    for (int64_t t = 0; t < T; t++) {
        residual_sum(x, residual, t, H, dtype, 1, s);
        float inv = inv_rms(s, H, 0, eps);
        for (int32_t i = 0; i < H; i++)
            st(x, t * H + i, dtype, apply_weight(s[i] * inv, w, i, dtype, weight_offset));
    }
    free(s);
    return 0;
}

int mbt_ref_fused_add_rmsnorm_fp8(const void* x, void* residual, const void* w,
                                  uint8_t* y, float inv_scale, int64_t T,
                                  int32_t H, float eps, int32_t weight_offset,
                                  int32_t dtype) {
    if (!norm_args_ok(w, T, H, weight_offset, dtype)) return -1;
    float* s = (float*)malloc((size_t)H * sizeof(float));
    if (!s) return -1;
    for (int64_t t = 0; t < T; t++) {
        residual_sum(x, residual, t, H, dtype, 1, s);
        float inv = inv_rms(s, H, 0, eps);
        for (int32_t i = 0; i < H; i++) {
            float v = fp8_source(apply_weight(s[i] * inv, w, i, dtype, weight_offset), dtype, 17);
            y[t * H + i] = mbt_ref_f32_to_e4m3fn(v * inv_scale);
        }
    }
    free(s);
    return 0;
}

float mbt_ref_fused_add_rmsnorm_amax(const void* x, const void* residual,
                                     const void* w, int64_t T, int32_t H,
                                     float eps, int32_t weight_offset,
                                     int32_t dtype) {
    if (!norm_args_ok(w, T, H, weight_offset, dtype)) return -1.0f;
    float* s = (float*)malloc((size_t)H * sizeof(float));
    if (!s) return -1;
    float amax = 0.0f;
    for (int64_t t = 0; t < T; t++) {
        residual_sum(x, (void*)residual, t, H, dtype, 0, s);
        float inv = inv_rms(s, H, 0, eps);
        for (int32_t i = 0; i < H; i++) {
            float v = magnitude(fp8_source(apply_weight(s[i] * inv, w, i, dtype,
                                                        weight_offset), dtype, 18));
            if (v > amax) amax = v;
        }
    }
    free(s);
    return amax;
}

/* ------------------------------------------------------------------------ */
/* Adaptive RMSNorm (FlashRT optimization details: the Pi0.5 decoder norms   */
/* are modulated by a style vector computed once per prompt; fused kernels    */
/* fused_adarms_fp8_static and gate_res_adarms_fp8_static).  The pages give  */
/* no formula; the reading taken: the style vector supplies per-channel      */
/* scale, shift and gate (each of length H) and                              */
/*   s = R(r + g * x)      (with a residual; g = 1 when no gate is given),   */
/*   s = x                 (without one),  r <- s,                           */
/*   m = (s * inv) * (1 + scale) + shift,  inv = 1 / sqrt(mean s^2 + eps),  */
/* each fp32 operation rounded as written, then R(m) or E4M3FN(m * inv_scale).*/
/* ------------------------------------------------------------------------ */

static void ada_sum(const void* x, void* residual, const void* gate, int64_t t, int32_t H,
                    int32_t dtype, int write_res, float* s) {
    for (int32_t i = 0; i < H; i++) {
        int64_t k = t * H + i;
        float xv = ld(x, k, dtype);
        if (residual) {
            float gx = gate ? ld(gate, i, dtype) * xv : xv;
#if MBT_ORACLE_MUTATION == 16
            gx = xv;                                  /* planted: gate ignored */
#endif
            float sum = ld(residual, k, dtype) + gx;
            s[i] = rounded(sum, dtype);
            if (write_res) st(residual, k, dtype, sum);
        } else {
            s[i] = xv;
        }
    }
}

static float modulate(float n, const void* scale, const void* shift, int32_t i, int32_t dtype) {
#if MBT_ORACLE_MUTATION == 15
    return n * ld(scale, i, dtype) + ld(shift, i, dtype); /* planted: 1 + scale lost */
#else
    return n * (1.0f + ld(scale, i, dtype)) + ld(shift, i, dtype);
#endif
}

static int ada_args_ok(const void* residual, const void* gate, const void* scale,
                       const void* shift, int64_t T, int32_t H, int32_t dtype) {
    return dtype_ok(dtype) && T >= 0 && H > 0 && scale && shift && (residual || !gate);
}

/* mode 0: x <- R(m); mode 1: y <- E4M3FN(m * inv_scale); mode 2: amax. */
static float adarms(void* x, void* residual, const void* gate, const void* scale,
                    const void* shift, uint8_t* y, float inv_scale, int64_t T, int32_t H,
                    float eps, int32_t dtype, int mode) {
    float* s = (float*)malloc((size_t)H * sizeof(float));
    if (!s) return -1.0f;
    float amax = 0.0f;
    for (int64_t t = 0; t < T; t++) {
        ada_sum(x, residual, gate, t, H, dtype, mode != 2, s);
        float inv = inv_rms(s, H, 0, eps);
        for (int32_t i = 0; i < H; i++) {
            float m = modulate(s[i] * inv, scale, shift, i, dtype);
            if (mode == 0) st(x, t * H + i, dtype, m);
            else if (mode == 1)
                y[t * H + i] = mbt_ref_f32_to_e4m3fn(fp8_source(m, dtype, 19) * inv_scale);
            else if (magnitude(fp8_source(m, dtype, 20)) > amax)
                amax = magnitude(fp8_source(m, dtype, 20));
        }
    }
    free(s);
    return amax;
}

int mbt_ref_adarms(void* x, void* residual, const void* gate, const void* scale,
                   const void* shift, int64_t T, int32_t H, float eps, int32_t dtype) {
    if (!ada_args_ok(residual, gate, scale, shift, T, H, dtype)) return -1;
    return adarms(x, residual, gate, scale, shift, NULL, 0.0f, T, H, eps, dtype, 0) < 0 ? -1 : 0;
}

int mbt_ref_adarms_fp8(const void* x, void* residual, const void* gate, const void* scale,
                       const void* shift, uint8_t* y, float inv_scale, int64_t T, int32_t H,
                       float eps, int32_t dtype) {
    if (!ada_args_ok(residual, gate, scale, shift, T, H, dtype)) return -1;
    return adarms((void*)x, residual, gate, scale, shift, y, inv_scale, T, H, eps, dtype, 1) < 0
               ? -1 : 0;
}

float mbt_ref_adarms_amax(const void* x, const void* residual, const void* gate,
                          const void* scale, const void* shift, int64_t T, int32_t H,
                          float eps, int32_t dtype) {
    if (!ada_args_ok(residual, gate, scale, shift, T, H, dtype)) return -1.0f;
    return adarms((void*)x, (void*)residual, gate, scale, shift, NULL, 0.0f, T, H, eps, dtype, 2);
}

/* ------------------------------------------------------------------------ */
/* Gated activations (P1 5.1): [g || u] in R^{2d}, out_j = act(g_j) * u_j.   */
/* SiLU(g) = g * sigmoid(g).                                                 */
/* GELU, tanh form: 0.5 g (1 + tanh(z)), z = sqrt(2/pi) (g + 0.044715 g^3).  */
/* Since 0.5 (1 + tanh z) = sigmoid(2z) exactly, GELU-tanh(g) = g sigmoid(2z)*/
/* and both activations reduce to one logistic function.                    */
/* ------------------------------------------------------------------------ */

/* sigmoid(x) = 1 / (1 + e^-x), evaluated through e^-|x| so that the
 * exponential never overflows and nothing cancels: the literal 1 + tanhf(z)
 * is 0 in fp32 for z < -9, and e^-g overflows for g < -88.7, while the true
 * values there are still representable in bf16. */
static float sigmoid(float x) {
    float e = expf(-fabsf(x));
    return x >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}

static float act_value(float g, int32_t act) {
#if MBT_ORACLE_MUTATION == 27
    if (act == MBT_REF_SILU) return g * sigmoid(-g);  /* planted: sigmoid of -g */
#endif
    if (act == MBT_REF_SILU) return g * sigmoid(g);
#if MBT_ORACLE_MUTATION == 7
    float z = 0.7978845608f * (g + 0.0447f * g * g * g);   /* planted */
#else
    float z = 0.7978845608f * (g + 0.044715f * g * g * g);
#endif
    return g * sigmoid(2.0f * z);
}

/* Offsets of g and u in a row of gate_up: the gate projection first. */
#if MBT_ORACLE_MUTATION == 23
#define GATE_OFF(d) ((int64_t)(d))                    /* planted: halves swapped */
#define UP_OFF(d) ((int64_t)0)
#else
#define GATE_OFF(d) ((int64_t)0)
#define UP_OFF(d) ((int64_t)(d))
#endif

/* The activation's value as the product consumes it: fp32, not rounded. */
static float act_operand(float a, int32_t dtype) {
#if MBT_ORACLE_MUTATION == 35
    return rounded(a, dtype);                         /* planted: act(g) rounded first */
#else
    (void)dtype;
    return a;
#endif
}

static int act_args_ok(int64_t T, int32_t d, int32_t act, int32_t dtype) {
    return dtype_ok(dtype) && T >= 0 && d > 0 &&
           (act == MBT_REF_SILU || act == MBT_REF_GELU_TANH);
}

int mbt_ref_gated_act(const void* gate_up, void* out, int64_t T, int32_t d,
                      int32_t act, int32_t dtype) {
    if (!act_args_ok(T, d, act, dtype)) return -1;
    for (int64_t t = 0; t < T; t++)
        for (int32_t j = 0; j < d; j++) {
            float g = ld(gate_up, t * 2 * (int64_t)d + GATE_OFF(d) + j, dtype);
            float u = ld(gate_up, t * 2 * (int64_t)d + UP_OFF(d) + j, dtype);
            st(out, t * (int64_t)d + j, dtype, act_operand(act_value(g, act), dtype) * u);
        }
    return 0;
}

int mbt_ref_gated_act_fp8(const void* gate_up, uint8_t* out, float inv_scale,
                          int64_t T, int32_t d, int32_t act, int32_t dtype) {
    if (!act_args_ok(T, d, act, dtype)) return -1;
    for (int64_t t = 0; t < T; t++)
        for (int32_t j = 0; j < d; j++) {
            float g = ld(gate_up, t * 2 * (int64_t)d + GATE_OFF(d) + j, dtype);
            float u = ld(gate_up, t * 2 * (int64_t)d + UP_OFF(d) + j, dtype);
            float v = fp8_source(act_operand(act_value(g, act), dtype) * u, dtype, 21);
            out[t * (int64_t)d + j] = mbt_ref_f32_to_e4m3fn(v * inv_scale);
        }
    return 0;
}

float mbt_ref_gated_act_amax(const void* gate_up, int64_t T, int32_t d,
                             int32_t act, int32_t dtype) {
    if (!act_args_ok(T, d, act, dtype)) return -1.0f;
    float amax = 0.0f;
    for (int64_t t = 0; t < T; t++)
        for (int32_t j = 0; j < d; j++) {
            float g = ld(gate_up, t * 2 * (int64_t)d + GATE_OFF(d) + j, dtype);
            float u = ld(gate_up, t * 2 * (int64_t)d + UP_OFF(d) + j, dtype);
            float v = magnitude(fp8_source(act_operand(act_value(g, act), dtype) * u, dtype, 22));
            if (v > amax) amax = v;
        }
    return amax;
}

int mbt_ref_quantize_fp8(const float* x, uint8_t* y, int64_t n, float inv_scale) {
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; i++) y[i] = mbt_ref_f32_to_e4m3fn(x[i] * inv_scale);
    return 0;
}
