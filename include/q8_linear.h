/*
 * q8_linear.h -- C ABI of the MI355X (gfx950) Q8_0 block-quantized weight linear.
 *
 * What is computed (sources are the pages describing the fucina engine):
 *   - "14. Model families and example applications", section 14.1 (Conventions shared
 *     by every family): LinearWeight keeps the GGUF dtype resident and the quant forms,
 *     Q8_0 among them, run packed kernels with no global dequantization at load; q/k/v
 *     are fused into one QKV matrix and gate/up into one gate_up matrix, one wider
 *     product per block.
 *   - Same page, section 14.2 (Qwen3 - dense and MoE): SwiGLU FFN; lockstep batch
 *     decode runs the trunk as one m = n pass that reads the weights once for all
 *     streams; the MoE FFN routes with softmax top-k (routerTopK, normalize_selected =
 *     norm_topk_prob) and runs the router-weighted SwiGLU mixture (moeSwiGluFfnSeq),
 *     grouped per expert, so that one pass over an expert's weights serves its tokens.
 *   - Same page, section 14.4 (Gemma 4 - text + MoE, "MoE expert kernels"): a
 *     counting-sort route plan and a per-token summation order kept fixed.
 *
 * Q8_0 tensor layout (the GGUF Q8_0 block; the pages name the format without spelling
 * it out): a row of length K is K/32 blocks of 34 bytes, each a little-endian IEEE
 * binary16 scale d followed by 32 signed 8-bit quants q; the weight is w = d * q.
 * Rows are contiguous: row n starts at byte n * (K/32) * 34.  Expert stacks are E such
 * matrices back to back.
 *
 * Conventions for every call below:
 *   - All tensor pointers are DEVICE pointers owned by the caller; nothing is freed,
 *     retained or allocated by the library.  Weights and inputs are only read.
 *   - Row-major float32 activations x [M][ldx] (the first K of each row used) and
 *     outputs [M][ld*].  Outputs are fully overwritten, never accumulated into.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls are
 *     asynchronous: they enqueue kernels and return; they never synchronize.
 *   - Arguments are validated on the host before anything is enqueued; on a bad
 *     argument the call returns an error code and enqueues nothing.  A launch failure
 *     reported by the HIP runtime returns Q8_ERR_DEVICE.  q8_last_error() then holds a
 *     thread-local description.
 *   - M = 0 (no rows) and N = 0 (no outputs) are valid and enqueue nothing.
 *   - K (and the MoE H and F) must be positive multiples of 256 (rows then stay 16-byte
 *     aligned: 8 blocks are 272 bytes); otherwise Q8_ERR_SHAPE.
 *   - Alignment: weight and x base pointers 16-byte aligned and ldx a multiple of 4;
 *     output pointers 4-byte aligned; otherwise Q8_ERR_ALIGN.
 *   - Results are deterministic: the same inputs give bit-identical outputs on every
 *     call (fixed summation orders, no floating-point atomics).
 *   - Calls are thread-safe; the only global state is the thread-local error text and
 *     a per-device cache of launch sizes.
 */
#ifndef Q8_LINEAR_H
#define Q8_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8_ABI_VERSION 8

typedef enum q8_status {
    Q8_OK = 0,
    Q8_ERR_NULL = 1,      /* a required pointer is NULL                                   */
    Q8_ERR_SHAPE = 2,     /* a size is negative, too large, or breaks the block structure */
    Q8_ERR_ALIGN = 3,     /* a pointer or leading dimension is misaligned                 */
    Q8_ERR_WORKSPACE = 4, /* workspace missing or smaller than q8_moe_workspace_bytes()   */
    Q8_ERR_DEVICE = 5     /* the HIP runtime reported an error                            */
} q8_status;

/* Version of this ABI (Q8_ABI_VERSION of the built library). */
int32_t q8_abi_version(void);

/* Static text for a status code. */
const char* q8_status_string(q8_status status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* q8_last_error(void);

/*
 * y = x . W^T  -- the packed-weight linear (section 14.1, LinearWeight; the fused QKV
 * and down projections use it directly).
 *   w_q8 : Q8_0 [n][k]          x : float32 [m][ldx]          y : float32 [m][ldy]
 *   n >= 0 outputs, k > 0 a multiple of 256, m >= 0 rows, ldx >= k, ldy >= n.
 * Arithmetic by batch size (the m-dependent kernel classes of section 14.2):
 *   m == 1      float32: per block t = sum q*x, acc = fma(d, t, acc), fixed butterfly;
 *   2..255      float32 in 16-row launches, per block t = sum q*x (the quants exact,
 *               one rounding per fma; the fp32 matrix cores' 4x4x1 form rounds like an
 *               fma), acc = fma(d, t, acc), in an order that depends only on k and n:
 *               k <= 4096 streams the weights once per launch on the matrix cores when
 *               its LDS fits (at k = 4096 on 256 CUs: n <= 129,024, fused f <= 47,104),
 *               a fixed sum over 16 pairs, then the 16-pair chunks in order; other calls
 *               run the float32 rows kernel (9..16 rows on its matrix-core form, the same
 *               bits); every row is bit-identical whatever the other rows are (for any m
 *               in 2..255), and agrees with the m == 1 result to reassociation;
 *   m >= 256    bf16 matrix cores (dense prefill): weights d*q and activations rounded
 *               to bf16 (nearest even), float32 accumulation and output.
 */
q8_status q8_linear(const void* w_q8, int64_t n, int64_t k,
                    const float* x, int64_t m, int64_t ldx,
                    float* y, int64_t ldy, void* stream);

/*
 * h = SiLU(x . W_gate^T) * (x . W_up^T) from one fused gate_up matrix (section 14.1 fuses
 * gate and up; section 14.2 gives the SwiGLU FFN).  SiLU(g) = g / (1 + exp(-g)).
 *   w_gate_up_q8 : Q8_0 [2f][k], gate rows [0, f) then up rows [f, 2f)
 *   x : float32 [m][ldx]          h : float32 [m][ldh], ldh >= f
 * Same rules (and the same arithmetic by batch size) as q8_linear otherwise.
 */
q8_status q8_linear_fused_gate_up_silu(const void* w_gate_up_q8, int64_t f, int64_t k,
                                       const float* x, int64_t m, int64_t ldx,
                                       float* h, int64_t ldh, void* stream);

/*
 * GGUF Q4_0 weights (the DGX Spark README, Features and Models: Q4_0 is read directly by
 * the quantized GEMV; section 14.1: the other ggml quant forms run their own packed
 * kernels).  The layout is the ggml one (the pages name the format only): per block of
 * 32 weights a little-endian binary16 scale d, then 16 bytes; weight j < 16 is the low
 * nibble of byte j, weight j + 16 the high nibble; w = d * (nibble - 8).  18 bytes per
 * block, rows of k/32 blocks back to back.
 *   q4_0_linear                     : y[m][n] = x . W^T,  W = Q4_0 [n][k]
 *   q4_0_linear_fused_gate_up_silu  : h = SiLU(x . W_gate^T) * (x . W_up^T), W = Q4_0 [2f][k]
 * Arguments, rules and errors as for q8_linear / q8_linear_fused_gate_up_silu.  Two or
 * more rows run the float32 rows kernel in 8-row launches (weights w = d*(q-8) exact in
 * float32, one fma per weight and row, the per-output order depends only on k: those rows
 * are bit-identical whatever m is).  One row with k <= 4096 on a matrix with at least 16
 * row groups per CU runs the one-row kernel (per block t = sum nibble*x, then
 * acc += d*(t - 8*sum x)), whose rows agree with the multi-row results to float32
 * reassociation; other one-row calls run the rows kernel.
 */
q8_status q4_0_linear(const void* w_q4_0, int64_t n, int64_t k,
                      const float* x, int64_t m, int64_t ldx,
                      float* y, int64_t ldy, void* stream);
q8_status q4_0_linear_fused_gate_up_silu(const void* w_gate_up_q4_0, int64_t f, int64_t k,
                                         const float* x, int64_t m, int64_t ldx,
                                         float* h, int64_t ldh, void* stream);

/*
 * GGUF k-quant weights, Q4_K, Q5_K and Q6_K ("14. Model families and example
 * applications", section 14.1: Q4_K, Q5_K and Q6_K run their own packed kernels; the DGX
 * Spark README, Features: the engine reads Q4_K and Q6_K blocks directly in its quantized
 * GEMV, without dequantizing the model at load).  The pages name the formats only; the
 * layouts are the ggml ones, super-blocks of 256 weights along k, rows of k/256
 * super-blocks back to back:
 *   Q4_K, 144 bytes: binary16 d, binary16 dmin, 12 bytes holding eight 6-bit (scale, min)
 *     pairs (sub-block j < 4: bits 0..5 of bytes j and j+4; j >= 4: the low / high
 *     nibble of byte j+4 below bits 6..7 of byte j-4 / j), 128 bytes of nibbles (weight
 *     64c+i is the low nibble of byte 32c+i, weight 64c+32+i its high nibble);
 *     w = d*sc*q - dmin*m for the weight's 32-wide sub-block.
 *   Q5_K, 176 bytes: the Q4_K header (d, dmin, 12 scale/min bytes), qh[32], then the
 *     Q4_K nibbles; weight 64c+32s+l (s < 2) gains 16 when bit 2c+s of qh[l] is set;
 *     w = d*sc*q - dmin*m with q in 0..31.
 *   Q6_K, 210 bytes: ql[128], qh[64], int8 scales[16], binary16 d; weight 128t+32u+l
 *     (t < 2, u < 4, l < 32) takes its low four bits from the low (u < 2) or high nibble
 *     of ql[64t + 32(u%2) + l] and its top two bits from bits 2u, 2u+1 of qh[32t + l];
 *     w = d * scales[weight/16] * (q - 32).
 *   q4_k_linear / q5_k_linear / q6_k_linear : y[m][n] = x . W^T, W [n][k]
 *   q4_k_/q5_k_/q6_k_linear_fused_gate_up_silu : h = SiLU(x . W_gate^T) * (x . W_up^T), W [2f][k]
 * Arguments, rules and errors as for q8_linear / q8_linear_fused_gate_up_silu (k a
 * positive multiple of 256, the weight base 16-byte aligned).  Two or more rows run the
 * float32 rows kernel in 8-row launches: weights are dequantized exactly in float32 (one
 * fma per weight), one fma per weight and row, and the per-output summation order depends
 * only on k, so those rows are bit-identical whatever m is.  One row runs the one-row
 * kernel when k <= 12288 (fused: k <= 8192; Q6_K: k <= 8192 and a multiple of 2048):
 * per 32-wide sub-block (Q6_K: 16-wide group) t = sum q*x, then acc += d*sc*t - dmin*m*sum x
 * (Q6_K: acc += d*s*(t - 32*sum x)), which agrees with the multi-row results to float32
 * reassociation; other one-row calls run the rows kernel.
 */
q8_status q4_k_linear(const void* w_q4_k, int64_t n, int64_t k,
                      const float* x, int64_t m, int64_t ldx,
                      float* y, int64_t ldy, void* stream);
q8_status q4_k_linear_fused_gate_up_silu(const void* w_gate_up_q4_k, int64_t f, int64_t k,
                                         const float* x, int64_t m, int64_t ldx,
                                         float* h, int64_t ldh, void* stream);
q8_status q5_k_linear(const void* w_q5_k, int64_t n, int64_t k,
                      const float* x, int64_t m, int64_t ldx,
                      float* y, int64_t ldy, void* stream);
q8_status q5_k_linear_fused_gate_up_silu(const void* w_gate_up_q5_k, int64_t f, int64_t k,
                                         const float* x, int64_t m, int64_t ldx,
                                         float* h, int64_t ldh, void* stream);
q8_status q6_k_linear(const void* w_q6_k, int64_t n, int64_t k,
                      const float* x, int64_t m, int64_t ldx,
                      float* y, int64_t ldy, void* stream);
q8_status q6_k_linear_fused_gate_up_silu(const void* w_gate_up_q6_k, int64_t f, int64_t k,
                                         const float* x, int64_t m, int64_t ldx,
                                         float* h, int64_t ldh, void* stream);

/*
 * Integer q8 x q8 path.  The DGX Spark README (Features; Architecture) names GEMV kernels
 * that read Q8_0 directly through int8 dot products, and the qwen3 runner README (q8_0 KV
 * cache; --cache-type) names an integer q8 x q8 dot path over quantized blocks.  No page
 * defines the activation code; the one used here:
 *   per block of 32 inputs, amax = max |x|;  dx = amax / 127;
 *   q = round-half-even(x * (127 / amax)) clamped to [-127, 127],
 *   each quotient and the product rounded to float32 (IEEE, subnormals kept);
 *   a block with amax < 2^-120 (an all-zero block among them) gets dx = 0 and q = 0.
 * Inputs must be finite (a NaN or infinity gives unspecified codes, never a fault).
 *
 * q8_quantize_act: codes and scales of float32 activation rows.
 *   x  : float32 [m][ldx], k > 0 a multiple of 256, ldx >= k (multiple of 4)
 *   xq : int8 [m][k] out, contiguous (row stride k bytes)
 *   xd : float32 [m][k/32] out, contiguous (row stride k/32)
 * x, xq and xd 16-byte aligned.  The result is bit-exact (a pure function of x).
 */
q8_status q8_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx,
                          int8_t* xq, float* xd, void* stream);

/*
 * y[t][n] = sum over blocks b of (d_w[n][b] * xd[t][b]) * sum_i q_w[n][b][i] * xq[t][b][i]
 * -- the packed-weight linear on int8 activation codes (any int8 value is accepted and
 * multiplied exactly; q8_quantize_act produces [-127, 127]).
 *   w_q8 : Q8_0 [n][k]     xq : int8 [m][k] contiguous     xd : float32 [m][k/32] contiguous
 *   y : float32 [m][ldy], ldy >= n
 * xq and xd 16-byte aligned; other rules as for q8_linear.  Block dot products are exact
 * 32-bit integers; per output, acc = fma(d_w * dx, float(isum), acc) over the blocks in a
 * fixed order that depends only on k, so every row is bit-identical whatever m is.
 */
q8_status q8_linear_q8act(const void* w_q8, int64_t n, int64_t k,
                          const int8_t* xq, const float* xd, int64_t m,
                          float* y, int64_t ldy, void* stream);

/* SiLU(gate) * up from one fused gate_up matrix [2f][k] on int8 activation codes (the
 * fused SwiGLU of q8_linear_fused_gate_up_silu with the arithmetic of q8_linear_q8act). */
q8_status q8_linear_fused_gate_up_silu_q8act(const void* w_gate_up_q8, int64_t f, int64_t k,
                                             const int8_t* xq, const float* xd, int64_t m,
                                             float* h, int64_t ldh, void* stream);

/*
 * Softmax top-k routing (section 14.2: routerTopK with normalize_selected =
 * norm_topk_prob, run on the device here instead of on the host).
 *   x        : float32 [m][ldx], hidden size h (h > 0 a multiple of 256, ldx >= h)
 *   w_router : float32 [n_exp][h], row-major, 1 <= n_exp <= 256
 *   k        : 1 <= k <= n_exp experts per token
 *   normalize: nonzero -> the chosen probabilities are divided by their sum
 *   topk_idx : int32 [m][k] out, descending probability, ties to the lower expert index
 *   topk_w   : float32 [m][k] out
 * Logits and the softmax are computed in float32.
 */
q8_status moe_route_topk(const float* x, int64_t m, int64_t h, int64_t ldx,
                         const float* w_router, int64_t n_exp, int32_t k, int32_t normalize,
                         int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Softmax top-k routing followed by adaptive expert top-p (section 14.2 Config:
 * moe_expert_top_p, 1.0 = full top-k; applyExpertTopP).  The pages give only the knob
 * and its neutral value; the cut used here: with the chosen probabilities p_j in
 * selection order, c_j their running float32 sum through slot j and S the sum over all
 * k slots, slot 0 is kept and slot j >= 1 while c_{j-1} < top_p * S; top_p = 1 keeps
 * all k (and then equals moe_route_topk bit for bit).  Kept weights are divided by the
 * kept sum when normalize is set; a dropped slot gets topk_idx = -1 and topk_w = 0,
 * which q8_moe_grouped_linear skips.
 *   top_p : in (0, 1], else Q8_ERR_SHAPE; other arguments as for moe_route_topk.
 */
q8_status moe_route_topk_top_p(const float* x, int64_t m, int64_t h, int64_t ldx,
                               const float* w_router, int64_t n_exp, int32_t k, int32_t normalize,
                               float top_p, int32_t* topk_idx, float* topk_w, void* stream);

/* Workspace bytes moe_route_topk_ws needs for m tokens and n_exp experts (0 on invalid sizes). */
size_t moe_route_workspace_bytes(int64_t m, int64_t n_exp);

/*
 * moe_route_topk_top_p in two passes that spread each token's logits over many CUs (one
 * kernel block per token is bound by one CU's load rate for the whole router matrix):
 * the logits go to the workspace, then one wave per token selects.  The logits are
 * summed in the same order as in the one-pass calls, so the results are bit-identical
 * to moe_route_topk_top_p (and to moe_route_topk when top_p = 1).
 *   workspace : device memory of at least moe_route_workspace_bytes(m, n_exp) bytes,
 *               16-byte aligned (Q8_ERR_WORKSPACE / Q8_ERR_ALIGN otherwise); its contents
 *               on entry do not matter and are overwritten.
 * Other arguments as for moe_route_topk_top_p.
 */
q8_status moe_route_topk_ws(const float* x, int64_t m, int64_t h, int64_t ldx,
                            const float* w_router, int64_t n_exp, int32_t k, int32_t normalize,
                            float top_p, int32_t* topk_idx, float* topk_w,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes q8_moe_grouped_linear needs for these sizes (0 on invalid sizes). */
size_t q8_moe_workspace_bytes(int64_t m, int32_t k, int64_t n_exp, int64_t f, int64_t h);

/*
 * Router-weighted SwiGLU expert mixture (section 14.2: moeSwiGluFfnSeq; section 14.4:
 * counting-sort route plan, fixed per-token summation order):
 *   y[t] = sum_{j=0..k-1} topk_w[t][j] * W_down[e] . (SiLU(W_gate[e] x_t) * (W_up[e] x_t)),
 *   e = topk_idx[t][j], summed in slot order j = 0, 1, ..., k-1.
 *   w_gate_up_exps : Q8_0 [n_exp][2f][h] (gate rows [0,f), up rows [f,2f) per expert)
 *   w_down_exps    : Q8_0 [n_exp][h][f]
 *   x : float32 [m][ldx] (ldx >= h)     y : float32 [m][ldy] (ldy >= h)
 *   topk_idx : int32 [m][k], entries in [0, n_exp), or -1 for a slot dropped by
 *              moe_route_topk_top_p (skipped: it contributes nothing; any other entry
 *              outside [0, n_exp) is skipped the same way, but is a caller error)
 *   topk_w   : float32 [m][k]
 *   workspace: device memory of at least q8_moe_workspace_bytes(m, k, n_exp, f, h)
 *              bytes, 256-byte aligned; its contents on entry do not matter.
 * Paths: below 8 routed pairs per expert on average (decode) the float32 GEMV passes run,
 * one pass over an expert's weights serving up to 4 of its routed tokens (an expert with
 * more tokens is streamed again for each further group of 4); from 8 pairs per expert on
 * average the bf16 matrix-core tiles run (activations, d*q and the hidden SiLU*up rounded
 * to bf16 once, float32 accumulation), one pass per 128 of an expert's tokens.  The
 * switch point is the measured crossover on the Qwen3-30B-A3B layer.
 */
q8_status q8_moe_grouped_linear(const void* w_gate_up_exps, const void* w_down_exps,
                                int64_t n_exp, int64_t f, int64_t h,
                                const float* x, int64_t m, int64_t ldx,
                                const int32_t* topk_idx, const float* topk_w, int32_t k,
                                float* y, int64_t ldy,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * q8_moe_grouped_linear without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The route plan and hidden
 * activations live in a fixed scratch array in device memory that the library holds
 * per device for the life of the process (Q8_MOE_NOALLOC_SCRATCH_BYTES, 16 MiB; about
 * 1170 routed (token, slot) pairs at the Qwen3-30B-A3B sizes f = 768, h = 2048).
 *   Arguments, arithmetic and results as q8_moe_grouped_linear (bit-identical outputs).
 *   Sizes whose workspace (q8_moe_workspace_bytes) exceeds the scratch are refused with
 *   Q8_ERR_WORKSPACE before anything is enqueued.  The first call on a device looks up
 *   the scratch's device address (a runtime query, no allocation).
 *   Every call on one device shares that device's scratch: calls that can overlap on one
 *   device (different streams, different host threads) race and must be serialized by
 *   the caller.  Nothing in the scratch needs to start at any value.
 */
#define Q8_MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
q8_status q8_moe_grouped_linear_noalloc(const void* w_gate_up_exps, const void* w_down_exps,
                                        int64_t n_exp, int64_t f, int64_t h,
                                        const float* x, int64_t m, int64_t ldx,
                                        const int32_t* topk_idx, const float* topk_w, int32_t k,
                                        float* y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8_LINEAR_H */
