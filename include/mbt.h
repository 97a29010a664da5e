/*
 * mbt.h -- C ABI of libmbt: fused memory-bound decoder ops for AMD Instinct
 * MI355X (gfx950).  ABI version 1.
 *
 * Pages cited below:
 *  [P1] "thox-edge-ops v2: fused decode kernels for small models on THOX edge
 *       hardware" (thox.ai preprint).
 *  [P2] ninfer PR #273, "Register the text profile of ops::rmsnorm_rope and
 *       route the two full-attention call sites to it".
 *  [P3] FlashRT "optimization details" (Pi0.5 on Jetson AGX Thor).
 *
 * Common rules for every entry point
 * ----------------------------------
 *  - Tensor pointers are DEVICE pointers (HBM) owned by the caller.  The
 *    library allocates nothing, performs no I/O and never synchronises the
 *    host (P1 section 5.5): every call enqueues its kernels on `stream` (a
 *    hipStream_t passed as void*, NULL = the null stream) and returns.
 *    Calls run on the current HIP device: `stream` must belong to it, and
 *    every pointer must be memory that device can address (its own HBM).
 *  - Tensors are dense, row-major, one element type per call:
 *    MBT_F32 (float), MBT_F16 (IEEE binary16), MBT_BF16 (bfloat16) -- the
 *    three dtypes of P1 section 3.  FP8 outputs are OCP e4m3fn codes (uint8).
 *  - Every value is decoded to fp32, all arithmetic and accumulation is fp32,
 *    and each output is rounded once to nearest-even (P1 section 3, R1).
 *  - All arguments are checked first, before the library computes an
 *    address or launches anything (P1 section 5.5); a rejected call
 *    enqueues nothing and returns the status below, with a detail string in
 *    mbt_last_error().  There is no fallback path: a configuration the
 *    kernels do not cover is an error.
 *  - T == 0 (no tokens / rows) is a successful no-op; NULL is an error only
 *    for a pointer the call needs when T > 0.
 *  - Any element-aligned pointer is accepted; 16-byte aligned, densely
 *    strided tensors take the vectorised kernels, others a scalar kernel
 *    with identical results.
 *  - Exact aliasing of an output with its input is the in-place form and is
 *    allowed where stated; any partial overlap between an input and an
 *    output (or between x and residual) is MBT_ERR_ALIAS.
 *  - Launch failures return MBT_ERR_HIP with the HIP error string in
 *    mbt_last_error(); faults during asynchronous execution surface at the
 *    caller's next synchronisation.
 *  - All entry points are thread-safe and reentrant.  Calls on one stream
 *    execute in order; calls on different streams that write the same
 *    memory race, as with any kernel.
 *  - Launch shapes (lanes and chunks per row, load order) are picked per
 *    call from the sizes, by thresholds fixed at compile time; the
 *    environment plays no part.  Every shape gives the same bits.
 */
#ifndef MBT_H
#define MBT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MBT_ABI_VERSION 1

#if defined(__GNUC__)
#define MBT_API __attribute__((visibility("default")))
#else
#define MBT_API
#endif

typedef enum {
    MBT_OK = 0,
    MBT_ERR_NULL_POINTER = 1, /* a required pointer is NULL                   */
    MBT_ERR_BAD_SHAPE = 2,    /* a size is negative, zero where it may not be, */
                              /* or outside the supported range                */
    MBT_ERR_BAD_DTYPE = 3,    /* dtype is not one of mbt_dtype                 */
    MBT_ERR_BAD_ENUM = 4,     /* layout / act / weight_offset out of range     */
    MBT_ERR_BAD_SCALAR = 5,   /* eps / inv_scale / max_pos not acceptable      */
    MBT_ERR_ALIAS = 6,        /* partial overlap of an input and an output     */
    MBT_ERR_HIP = 7,          /* the HIP runtime reported an error             */
    MBT_ERR_ALIGN = 8         /* a pointer is not aligned to its element size  */
} mbt_status;

typedef enum { MBT_F32 = 0, MBT_F16 = 1, MBT_BF16 = 2 } mbt_dtype;

/* Rotary pairings (P1 section 2 and section 5.1): rotate-half pairs channel
 * i with i + rot_dim/2 (GPT-NeoX lineage); interleaved pairs 2i with 2i+1
 * (GPT-J lineage); i < rot_dim/2 in both. */
typedef enum { MBT_ROPE_ROTATE_HALF = 0, MBT_ROPE_INTERLEAVED = 1 } mbt_rope_layout;

/* Gated activations on [g || u] (P1 section 5.1): SiLU (Llama / Qwen MLP)
 * and the tanh approximation of GELU (Gemma MLP). */
typedef enum { MBT_ACT_SILU = 0, MBT_ACT_GELU_TANH = 1 } mbt_act;

/* Flags of mbt_qknorm_rope_ex and mbt_qkv_norm_rope_cache.
 * MBT_QK_ROUND_ONCE: the single-rounding variant (P2, review item 1): the
 * first rot_dim channels are rotated from the fp32 norm result and rounded
 * once, after the rotation, instead of rotating the rounded norm result. */
#define MBT_QK_ROUND_ONCE 1

/*
 * mbt_qknorm_rope -- fused per-head QK-RMSNorm + rotary embedding prologue.
 *
 * Defined by P1 section 5.1 (last paragraph) and section 5.4, and by P2
 * "Implementation": each query head is RMS-normalised with w_q and each key
 * head with w_k (weights of length head_dim), the normalised value is rounded
 * to the I/O dtype, and that rounded value is rotated:
 *   inv   = 1 / sqrt(mean_{i<head_dim} x_i^2 + eps)
 *   n_i   = R((x_i * inv) * (w_i + weight_offset))          (all channels)
 *   for each pair (a, b) of the first rot_dim channels, with c = cos_sin[p][j],
 *   s = cos_sin[p][rot_dim/2 + j] (j the pair index):
 *   out_a = R(n_a c - n_b s),  out_b = R(n_b c + n_a s)
 *   channels >= rot_dim: out = n.
 * A token whose position p = pos[t] lies outside [0, max_pos) is normalised
 * but not rotated (P1 section 5.4; R5: the cache is never read past its end).
 *
 *  q_in   [T][Q][head_dim]  dtype      query heads (read)
 *  k_in   [T][K][head_dim]  dtype      key heads (read)
 *  q_out  [T][Q][head_dim]  dtype      written; may equal q_in (in place)
 *  k_out  [T][K][head_dim]  dtype      written; may equal k_in (in place)
 *  w_q, w_k  [head_dim]     dtype      norm weights; weight_offset 0 applies
 *                                      w (Llama/Qwen3), 1 applies 1 + w formed
 *                                      in fp32 (Gemma; P2's text profile)
 *  cos_sin  [max_pos][rot_dim] fp32    caller-built cache: cos in columns
 *                                      [0, rot_dim/2), sin in [rot_dim/2, rot_dim)
 *  pos    [T] int64                    position of each token
 *  Q, K   0 .. 2^20, Q + K >= 1        heads per token
 *  T      >= 0                         tokens
 *  head_dim 1..512; rot_dim even, 0..head_dim; eps finite, >= 0;
 *  max_pos >= 0; weight_offset in {0,1}; layout mbt_rope_layout; dtype mbt_dtype.
 * w_k may be NULL when K == 0, w_q when Q == 0; cos_sin may be NULL when
 * rot_dim == 0 or max_pos == 0.
 */
MBT_API mbt_status mbt_qknorm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                           const void* w_q, const void* w_k,
                           const float* cos_sin, int64_t max_pos, const int64_t* pos,
                           int32_t Q, int32_t K, int64_t T, int32_t head_dim,
                           int32_t rot_dim, float eps, int32_t weight_offset,
                           int32_t layout, int32_t dtype, void* stream);

/*
 * mbt_qknorm_rope_ex -- mbt_qknorm_rope on strided views, with flags.
 *
 * The same operation as mbt_qknorm_rope (flags 0), or its single-rounding
 * variant (flags MBT_QK_ROUND_ONCE, P2 review item 1):
 *   out_a = R(n'_a c - n'_b s),  out_b = R(n'_b c + n'_a s),
 *   n'_i = (x_i * inv) * (w_i + weight_offset) in fp32, not rounded;
 *   channels >= rot_dim and tokens outside the cache: R(n'_i) as before.
 * Each tensor may be a strided view (P1 section 6: strided views, as when q
 * and k are slices of one fused QKV projection buffer): the heads of one
 * token are contiguous ([heads][head_dim]) and consecutive tokens are
 * *_stride elements apart.
 *
 *  q_in_stride, k_in_stride, q_out_stride, k_out_stride
 *         token strides in elements; 0 = dense (Q * head_dim or
 *         K * head_dim); otherwise >= that and <= 2^40
 *  flags  0 or MBT_QK_ROUND_ONCE
 *  everything else: as for mbt_qknorm_rope.
 * An output may be the very view of the input it replaces (in place, same
 * pointer and stride); any other overlap of an output with an input or with
 * the other output is MBT_ERR_ALIAS (views with equal strides are compared
 * row by row, so q and k slices of one buffer may be updated in place).
 * Alignment: element-aligned pointers and any stride; 16-byte aligned
 * pointers and strides take the vector kernel.
 */
MBT_API mbt_status mbt_qknorm_rope_ex(const void* q_in, const void* k_in, void* q_out,
                                      void* k_out, const void* w_q, const void* w_k,
                                      const float* cos_sin, int64_t max_pos,
                                      const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                                      int32_t head_dim, int32_t rot_dim, float eps,
                                      int32_t weight_offset, int32_t layout, int32_t dtype,
                                      int64_t q_in_stride, int64_t k_in_stride,
                                      int64_t q_out_stride, int64_t k_out_stride, int32_t flags,
                                      void* stream);

/*
 * mbt_qkv_norm_rope_cache -- the prologue on a fused QKV buffer with the
 * key / value cache write fused in.
 *
 * P3's decoder kernel list (qkv_split_rope_kvcache: split Q/K/V, rotary
 * embedding and the KV cache write in one kernel) and P1 section 10 (a KV
 * write fused into the prologue), with the per-head norm of
 * mbt_qknorm_rope: for every token t,
 *   q_out[t]            <- the prologue's query heads of qkv[t][0 : Q]
 *   k_cache[slot[t]]    <- the prologue's key heads of qkv[t][Q : Q + K]
 *   v_cache[slot[t]]    <- qkv[t][Q + K : Q + 2K], copied unchanged
 * A slot outside [0, n_slots) (e.g. -1 for padding) writes no cache row; the
 * token's q_out row is still written.  Valid tokens should map to distinct
 * slots.  Tokens that share one race for its row: the call still succeeds,
 * every element of that row ends up holding the element of one of those
 * tokens, and which token's element lands is unspecified (it may differ
 * from element to element).  The library does not check for shared slots,
 * since that would need the slot table on the host.
 *
 *  qkv      [T][Q + 2K][head_dim]  dtype  read
 *  q_out    [T][Q][head_dim]       dtype  written (may be NULL when Q == 0)
 *  k_cache, v_cache [n_slots][K][head_dim] dtype  rows written at the slots
 *  slot     [T] int64                     cache row of each token
 *  n_slots  >= 0
 *  K >= 1; Q >= 0; flags 0 or MBT_QK_ROUND_ONCE; everything else as for
 *  mbt_qknorm_rope.  No output may overlap qkv, the weights, the cache of
 *  angles, pos, slot or another output.
 */
MBT_API mbt_status mbt_qkv_norm_rope_cache(const void* qkv, void* q_out, void* k_cache,
                                           void* v_cache, const int64_t* slot, int64_t n_slots,
                                           const void* w_q, const void* w_k,
                                           const float* cos_sin, int64_t max_pos,
                                           const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                                           int32_t head_dim, int32_t rot_dim, float eps,
                                           int32_t weight_offset, int32_t layout, int32_t dtype,
                                           int32_t flags, void* stream);

/*
 * mbt_rope -- standalone rotary position embedding, in place.
 *
 * P1 section 5.1 (rotary embedding of every query and key head by the angles
 * cached for the token's position) and section 3 R5 (a position outside the
 * cache leaves that token untouched): for each token t with
 * 0 <= p = pos[t] < max_pos, each pair (a, b) of the first rot_dim channels
 * of every head (rotate-half: (j, j + rot_dim/2); interleaved: (2j, 2j+1)) is
 *   a <- R(a c - b s),  b <- R(b c + a s),  c = cos_sin[p][j],
 *   s = cos_sin[p][rot_dim/2 + j],
 * each product rounded on its own; other channels and out-of-range tokens are
 * not written.  Together with mbt_fused_add_rmsnorm (residual = NULL) on the
 * head rows it is the three-call route the fused prologue replaces, and it
 * reproduces mbt_qknorm_rope bit for bit.
 *
 *  q [T][Q][head_dim], k [T][K][head_dim]  dtype, read and written in place;
 *                                          must not overlap each other
 *  cos_sin, pos, max_pos, Q, K, T, head_dim, rot_dim, layout, dtype: as for
 *  mbt_qknorm_rope.
 */
MBT_API mbt_status mbt_rope(void* q, void* k, const float* cos_sin, int64_t max_pos,
                            const int64_t* pos, int32_t Q, int32_t K, int64_t T,
                            int32_t head_dim, int32_t rot_dim, int32_t layout, int32_t dtype,
                            void* stream);

/*
 * mbt_fused_add_rmsnorm -- residual add + RMSNorm in one pass, in place.
 *
 * Defined by P1 section 5.1 (the residual sum is stored back into the
 * residual stream, and it is that stored, already rounded sum which gets
 * normalised, all within one kernel) and R1 (the stored sum must match an
 * eager elementwise add bit for bit):
 *   s_i = R(x_i + r_i)        fp32 add of the two decoded values, rounded once
 *   residual_i <- s_i
 *   x_i <- R((s_i * inv) * (w_i + weight_offset)),  inv = 1/sqrt(mean s^2 + eps)
 * residual == NULL: s = x and only x is written (plain RMSNorm of each row).
 *
 *  x        [T][H] dtype  read, then overwritten with the normalised row
 *  residual [T][H] dtype  read, then overwritten with s; may be NULL; must
 *                         not overlap x
 *  w        [H]    dtype  norm weight; may be NULL: no weight multiply,
 *                         x_i <- R(s_i * inv) (P3, weight folding: the scale
 *                         is folded into the next GEMM's weight at load
 *                         time), and then weight_offset must be 0
 *  T >= 0; 1 <= H <= 2^28 (any width, odd included); eps finite >= 0;
 *  weight_offset in {0,1}; dtype mbt_dtype.
 *  Errors: NULL x (T > 0), or NULL w with weight_offset 1 -> NULL_POINTER.
 */
MBT_API mbt_status mbt_fused_add_rmsnorm(void* x, void* residual, const void* w, int64_t T,
                                 int32_t H, float eps, int32_t weight_offset,
                                 int32_t dtype, void* stream);

/*
 * mbt_fused_add_rmsnorm_fp8 -- the same step with static-scale FP8 output.
 *
 * P3, fused kernel table (rms_norm_fp8_static, residual_add_rms_norm_fp8_static)
 * and the static FP8 calibration paragraph: the normalised value is quantized
 * in the same pass with a scale fixed ahead of time, instead of an amax
 * reduction and a separate quantize kernel.
 *   y_i = E4M3FN(((s_i * inv) * (w_i + weight_offset)) * inv_scale)
 * E4M3FN rounds to nearest-even and saturates to +-448; a NaN gives a NaN
 * code (0xFF on gfx950, whatever the input NaN's sign).
 *
 *  x        [T][H] dtype  read only
 *  residual [T][H] dtype  read, then overwritten with s; may be NULL
 *  w        [H]    dtype  may be NULL (no weight, weight_offset 0): the
 *                         rms_norm_fp8_noweight form of P3's weight folding
 *  y        [T][H] uint8  e4m3fn codes, written; must not overlap the inputs
 *  inv_scale finite, > 0 (e.g. 448 / calibration amax)
 */
MBT_API mbt_status mbt_fused_add_rmsnorm_fp8(const void* x, void* residual, const void* w,
                                     uint8_t* y, float inv_scale, int64_t T, int32_t H,
                                     float eps, int32_t weight_offset, int32_t dtype,
                                     void* stream);

/*
 * mbt_fused_add_rmsnorm_amax -- calibration pass of the FP8 variant (P3,
 * static FP8 calibration: one forward pass measures the amax of each
 * quantization point).  Computes max |(s_i * inv) * (w_i + weight_offset)|
 * over all T x H values and folds it into *amax: *amax <- max(*amax, that).
 * Nothing else is written (the residual is NOT updated).  The caller
 * initialises *amax (a device float, >= 0), e.g. to 0.  w may be NULL, as for
 * the FP8 variant.
 */
MBT_API mbt_status mbt_fused_add_rmsnorm_amax(const void* x, const void* residual, const void* w,
                                      float* amax, int64_t T, int32_t H, float eps,
                                      int32_t weight_offset, int32_t dtype, void* stream);

/*
 * mbt_adarms, mbt_adarms_fp8, mbt_adarms_amax -- adaptive RMSNorm with a
 * per-call style vector.
 *
 * P3, fused kernel table (fused_adarms_fp8_static, gate_res_adarms_fp8_static)
 * and the style-vector paragraph: the Pi0.5 decoder norms are modulated by a
 * vector computed once per prompt.  The pages give no formula; the library
 * takes the style vector as per-channel scale, shift and gate and computes
 *   s_i = R(r_i + g_i * x_i)   with a residual (g = 1 when gate is NULL;
 *                              the product and the sum rounded in fp32, then
 *                              once to the dtype), s = x without one
 *   residual_i <- s_i
 *   m_i = (s_i * inv) * (1 + scale_i) + shift_i,  inv = 1/sqrt(mean s^2 + eps)
 * mbt_adarms:      x_i <- R(m_i)                         (in place)
 * mbt_adarms_fp8:  y_i = E4M3FN(m_i * inv_scale)        (x read only)
 * mbt_adarms_amax: *amax <- max(*amax, max |m_i|); nothing else written
 *
 *  x        [T][H] dtype
 *  residual [T][H] dtype  may be NULL; read, then overwritten with s (not by
 *                         the amax pass)
 *  gate     [H]    dtype  may be NULL; needs a residual
 *  scale, shift [H] dtype required
 *  y        [T][H] uint8  e4m3fn codes;  amax: device float, caller-initialised
 *  T >= 0; H >= 1; eps finite >= 0; inv_scale finite > 0; dtype mbt_dtype.
 *  Errors: a gate without a residual, or a NULL scale / shift / y / amax
 *  (T > 0) -> MBT_ERR_NULL_POINTER; overlaps of an output with an input ->
 *  MBT_ERR_ALIAS.
 */
MBT_API mbt_status mbt_adarms(void* x, void* residual, const void* gate, const void* scale,
                              const void* shift, int64_t T, int32_t H, float eps, int32_t dtype,
                              void* stream);
MBT_API mbt_status mbt_adarms_fp8(const void* x, void* residual, const void* gate,
                                  const void* scale, const void* shift, uint8_t* y,
                                  float inv_scale, int64_t T, int32_t H, float eps, int32_t dtype,
                                  void* stream);
MBT_API mbt_status mbt_adarms_amax(const void* x, const void* residual, const void* gate,
                                   const void* scale, const void* shift, float* amax, int64_t T,
                                   int32_t H, float eps, int32_t dtype, void* stream);

/*
 * mbt_gated_act -- gated activation (P1 section 5.1: the input row is the
 * gate projection followed by the up projection, [g || u] of width 2d):
 *   out[t][j] = R(act(g) * u),  g = gate_up[t][j],  u = gate_up[t][d + j]
 *   SiLU(g) = g * sigmoid(g);  GELU-tanh(g) = g * sigmoid(2z),
 *   z = sqrt(2/pi) (g + 0.044715 g^3)  (= 0.5 g (1 + tanh z)).
 *
 *  gate_up [T][2d] dtype  read
 *  out     [T][d]  dtype  written; must not overlap gate_up
 *  T >= 0; 1 <= d <= 2^28; act mbt_act; dtype mbt_dtype.
 */
MBT_API mbt_status mbt_gated_act(const void* gate_up, void* out, int64_t T, int32_t d,
                         int32_t act, int32_t dtype, void* stream);

/*
 * mbt_gated_act_fp8 -- the same with static-scale FP8 output (P3, fused
 * kernel table: gate_geglu_merged_fp8; packed-store row of the kernel-level
 * table):  out[t][j] = E4M3FN((act(g) * u) * inv_scale).
 *  out [T][d] uint8 e4m3fn codes; inv_scale finite, > 0.
 */
MBT_API mbt_status mbt_gated_act_fp8(const void* gate_up, uint8_t* out, float inv_scale,
                             int64_t T, int32_t d, int32_t act, int32_t dtype,
                             void* stream);

/*
 * mbt_gated_act_amax -- calibration pass of mbt_gated_act_fp8:
 * *amax <- max(*amax, max |act(g) * u|).  The caller initialises *amax.
 */
MBT_API mbt_status mbt_gated_act_amax(const void* gate_up, float* amax, int64_t T, int32_t d,
                              int32_t act, int32_t dtype, void* stream);

/*
 * mbt_quantize_fp8 -- standalone static quantization (P3, decoder kernel
 * list: quantize_fp8_static): y_i = E4M3FN(x_i * inv_scale) for n fp32
 * values.  Uses the same conversion as the fused FP8 epilogues.
 *  x [n] fp32 read; y [n] uint8 written, must not overlap x; n >= 0.
 */
MBT_API mbt_status mbt_quantize_fp8(const float* x, uint8_t* y, int64_t n, float inv_scale,
                            void* stream);

/*
 * mbt_stream_copy -- calibration, not a step of the method: copies nbytes
 * from src to dst with the streaming (nontemporal) 16-byte loads and stores
 * the kernels above use, chunks_per_lane 16-byte chunks per lane, all loads
 * of a lane before its first store; with block_sync = 1 every load of a
 * 256-lane block lands before any of its stores (a block barrier).  A memory-bound kernel pays a DRAM read,
 * a DRAM write and a launch (P3, the overview of its fused ops); this copy
 * pays only those, so the fastest chunks_per_lane at a byte count is the
 * floor a fused kernel moving that many bytes is measured against.
 *  src [nbytes] read; dst [nbytes] written; must not overlap at all.
 *  0 <= nbytes <= 2^40, a multiple of 16 (MBT_ERR_BAD_SHAPE); src and dst
 *  16-byte aligned (MBT_ERR_ALIGN); chunks_per_lane 1, 2, 4 or 8 and
 *  block_sync 0 or 1 (MBT_ERR_BAD_ENUM).  nbytes == 0 is a no-op.
 */
MBT_API mbt_status mbt_stream_copy(const void* src, void* dst, int64_t nbytes,
                                   int32_t chunks_per_lane, int32_t block_sync,
                                   void* stream);

/* Human-readable name of a status. */
MBT_API const char* mbt_status_string(mbt_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
MBT_API const char* mbt_last_error(void);

/* MBT_ABI_VERSION of the loaded library. */
MBT_API int32_t mbt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MBT_H */
