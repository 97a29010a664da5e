/*
 * mbt_oracle.h -- plain, single-threaded CPU oracle for the fused
 * memory-bound decoder ops.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the HIP path: the
 * dtype codes, layout codes and converters below are written out again here
 * on purpose.
 *
 * All pointers are HOST pointers.  Tensors are dense row-major.  16-bit
 * element types (bf16, fp16) are passed as their raw uint16 bit patterns,
 * fp32 as float, e4m3fn as uint8 codes.
 *
 * Arithmetic follows the numerics requirement of "thox-edge-ops v2: fused
 * decode kernels for small models on THOX edge hardware" (section 3, R1):
 * every value is decoded exactly to fp32, all arithmetic and accumulation is
 * IEEE fp32 in index order (compiled with -ffp-contract=off so no product is
 * fused), and each output is rounded once, to nearest-even, to its dtype.
 *
 * Every function returns 0 on success and -1 on an argument it does not
 * accept (it does not try to reproduce the library's status codes).
 */
#ifndef MBT_ORACLE_H
#define MBT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes (same numbering as the library's ABI, restated here) */
#define MBT_REF_F32  0
#define MBT_REF_F16  1
#define MBT_REF_BF16 2

/* rotary layouts */
#define MBT_REF_ROTATE_HALF 0   /* pairs (i, i + rot/2), GPT-NeoX lineage */
#define MBT_REF_INTERLEAVED 1   /* pairs (2i, 2i + 1), GPT-J lineage       */

/* gated activations */
#define MBT_REF_SILU      0
#define MBT_REF_GELU_TANH 1

/* ---- scalar converters (exposed so the tests can pin them) ------------- */
float    mbt_ref_bf16_to_f32(uint16_t h);
uint16_t mbt_ref_f32_to_bf16(float f);
float    mbt_ref_f16_to_f32(uint16_t h);
uint16_t mbt_ref_f32_to_f16(float f);
float    mbt_ref_e4m3fn_to_f32(uint8_t c);
uint8_t  mbt_ref_f32_to_e4m3fn(float f);

/* bulk versions of the converters: n elements */
void mbt_ref_encode(const float* in, void* out, int64_t n, int32_t dtype);
void mbt_ref_decode(const void* in, float* out, int64_t n, int32_t dtype);
void mbt_ref_encode_e4m3fn(const float* in, uint8_t* out, int64_t n);
void mbt_ref_decode_e4m3fn(const uint8_t* in, float* out, int64_t n);

/* ---- row primitives ---------------------------------------------------- */

/* RMSNorm of `rows` independent rows of width D (thox-edge-ops v2, 5.1):
 * y = R((x * inv) * (w + delta)), inv = 1 / sqrt(sum(x^2)/D + eps).
 * y may alias x exactly.  In this and the fused norms below, w == NULL means
 * no weight (FlashRT optimization details, weight folding): y = R(x * inv),
 * and then weight_offset must be 0. */
int mbt_ref_rmsnorm_rows(const void* x, void* y, const void* w, int64_t rows,
                         int32_t D, float eps, int32_t weight_offset,
                         int32_t dtype);

/* Standalone rotary embedding, in place, on x[T][heads][D]
 * (thox-edge-ops v2, 5.1 and R5): rotates the first rot_dim channels of every
 * head of token t by the cached angles of position pos[t]; a position outside
 * [0, max_pos) is skipped: its values are not modified. */
int mbt_ref_rope(void* x, const float* cos_sin, int64_t max_pos,
                 const int64_t* pos, int64_t T, int32_t heads, int32_t D,
                 int32_t rot_dim, int32_t layout, int32_t dtype);

/* ---- the operations on the path ---------------------------------------- */

/* Fused per-head QK-RMSNorm + RoPE prologue (thox-edge-ops v2, 5.1 and 5.4;
 * ninfer PR #273, "Implementation").  q_in [T][Q][D], k_in [T][K][D];
 * outputs of the same shapes; q_out may equal q_in and k_out may equal k_in.
 * cos_sin is fp32 [max_pos][rot_dim]: cos in [0, rot/2), sin in [rot/2, rot). */
int mbt_ref_qknorm_rope(const void* q_in, const void* k_in, void* q_out,
                        void* k_out, const void* w_q, const void* w_k,
                        const float* cos_sin, int64_t max_pos,
                        const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                        int32_t head_dim, int32_t rot_dim, float eps,
                        int32_t weight_offset, int32_t layout, int32_t dtype);

/* Single-rounding variant of the prologue (ninfer PR #273, review item 1):
 * the first rot_dim channels are rotated from the fp32 norm result and
 * rounded once, after the rotation; the other channels are as above. */
int mbt_ref_qknorm_rope_round_once(const void* q_in, const void* k_in, void* q_out,
                                   void* k_out, const void* w_q, const void* w_k,
                                   const float* cos_sin, int64_t max_pos,
                                   const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                                   int32_t head_dim, int32_t rot_dim, float eps,
                                   int32_t weight_offset, int32_t layout, int32_t dtype);

/* Fused residual-add RMSNorm, in place (thox-edge-ops v2, 5.1):
 * s = R(x + r); r <- s; x <- R((s * inv) * (w + delta)).
 * residual == NULL: s = x and only x is written. */
int mbt_ref_fused_add_rmsnorm(void* x, void* residual, const void* w,
                              int64_t T, int32_t H, float eps,
                              int32_t weight_offset, int32_t dtype);

/* Same, with the output quantized to OCP e4m3fn by a static scale
 * (FlashRT optimization details, fused kernel table and static FP8
 * calibration): residual in place, x read only, y[T][H] e4m3fn codes of
 * (s * inv) * (w + delta) * inv_scale. */
int mbt_ref_fused_add_rmsnorm_fp8(const void* x, void* residual, const void* w,
                                  uint8_t* y, float inv_scale, int64_t T,
                                  int32_t H, float eps, int32_t weight_offset,
                                  int32_t dtype);

/* Adaptive RMSNorm with a per-call style vector (FlashRT optimization
 * details: fused_adarms_fp8_static, gate_res_adarms_fp8_static).  Reading:
 *   s = R(r + g * x) with a residual (g = 1 when gate is NULL), else s = x;
 *   r <- s;  m = (s * inv) * (1 + scale) + shift.
 * scale, shift, gate: [H] in the dtype; a gate needs a residual.
 * mbt_ref_adarms writes x <- R(m); the _fp8 form writes y = E4M3FN(m *
 * inv_scale) and leaves x alone; _amax returns max |m| and writes nothing. */
int mbt_ref_adarms(void* x, void* residual, const void* gate, const void* scale,
                   const void* shift, int64_t T, int32_t H, float eps, int32_t dtype);
int mbt_ref_adarms_fp8(const void* x, void* residual, const void* gate, const void* scale,
                       const void* shift, uint8_t* y, float inv_scale, int64_t T, int32_t H,
                       float eps, int32_t dtype);
float mbt_ref_adarms_amax(const void* x, const void* residual, const void* gate,
                          const void* scale, const void* shift, int64_t T, int32_t H,
                          float eps, int32_t dtype);

/* Gated activation on gate_up[T][2d] = [g || u] (thox-edge-ops v2, 5.1):
 * out[t][j] = R(act(g_j) * u_j). */
int mbt_ref_gated_act(const void* gate_up, void* out, int64_t T, int32_t d,
                      int32_t act, int32_t dtype);

/* Same, quantized to e4m3fn with a static scale (FlashRT, GELU + gate + FP8). */
int mbt_ref_gated_act_fp8(const void* gate_up, uint8_t* out, float inv_scale,
                          int64_t T, int32_t d, int32_t act, int32_t dtype);

/* Standalone static quantization of fp32 values to e4m3fn. */
int mbt_ref_quantize_fp8(const float* x, uint8_t* y, int64_t n,
                         float inv_scale);

/* Calibration pass (FlashRT, static FP8 calibration): the largest magnitude
 * of the fp32 values the FP8 variants would quantize, before any scale. */
float mbt_ref_fused_add_rmsnorm_amax(const void* x, const void* residual,
                                     const void* w, int64_t T, int32_t H,
                                     float eps, int32_t weight_offset,
                                     int32_t dtype);
float mbt_ref_gated_act_amax(const void* gate_up, int64_t T, int32_t d,
                             int32_t act, int32_t dtype);

#ifdef __cplusplus
}
#endif
#endif
