/*
 * jepa_mi355x_ops.h -- the encoder's individual kernels, on caller-owned
 * device buffers.  The same kernels jepa_encode launches, exposed one by one
 * for kernel-level tests and measurements.  Conventions as in jepa_mi355x.h:
 * a jepa_status return, arguments validated before anything is enqueued,
 * work enqueued on the given HIP stream (NULL = default stream).
 */
#ifndef JEPA_MI355X_OPS_H
#define JEPA_MI355X_OPS_H

#include "jepa_mi355x.h"

/* Position of token n within a row of the transposed-V layout (vt) that
 * jepa_op_gemm_qkv and jepa_op_transpose_v write and jepa_op_attention reads:
 * bits 2 and 3 of n swapped, i.e. each aligned run of 16 tokens in the order
 * 0-3, 8-11, 4-7, 12-15. */
#define JEPA_VT_POS(n) (((n) & ~(int64_t)12) | (((n) & 4) << 1) | (((n) & 8) >> 1))

/* log2(e) / sqrt(64).  q multiplied by it turns q.k into the base-2 exponent
 * of the softmax (scale 1/sqrt(head_dim), base e); jepa_encode folds it into
 * the qkv layer's q columns (q_scale) and runs attention with q_prescaled. */
#define JEPA_ATTN_Q_SCALE 0.18033688011112042f

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JEPA_EPI_STORE = 0,   /* out[m, n] = act(acc + bias[n]) */
    JEPA_EPI_GELU = 1,    /* out[m, n] = act(gelu_erf(acc + bias[n])) */
    JEPA_EPI_RESID = 2    /* out[m, n] += acc + bias[n], out f32 */
} jepa_epilogue;

/* Pixel ingest (pages: a seeded uint8 stream through the model's own
 * normalisation -- benchmarks page, "Box and build"; tubelet tokens -- V-JEPA 2
 * card, opening paragraph).  frames uint8 [batch, frames, img_h, img_w, 3]
 * -> out act [batch*Np, ld], row = slot-major raster token, columns
 * (dt, dy, dx, c) with c fastest, value (u/255 - mean[c])/std[c]; columns
 * P..ld-1 zero.  ld >= P. */
jepa_status jepa_op_patchify(int act_dtype, const uint8_t *frames, int batch, int frames_per_item,
                             int img_h, int img_w, int tubelet, int patch, const float mean[3],
                             const float std[3], void *out, int64_t ld, void *hip_stream);

/* LayerNorm (pre-LN blocks and the final norm; the Quantization page names
 * ln1 / ln2 / norm): y = (x - mean)/sqrt(var + eps)*gamma + beta per row,
 * biased variance.  x, gamma, beta f32 device; y dtype y_dtype (F32, F16,
 * BF16), [rows, dim]. */
jepa_status jepa_op_layernorm(const float *x, int64_t rows, int dim, const float *gamma,
                              const float *beta, float eps, void *y, int y_dtype, void *hip_stream);

/* Linear layer (attn_qkv / attn_out / ffn_up / ffn_down, Quantization page
 * "The rule"): acc = a[M, K] * w[N, K]^T in f32, then the epilogue.  a is
 * act_dtype; w is act_dtype (dense) or packed Q8_0 / Q4_0 (see
 * jepa_pack_blocks) with w_scale its f16 scales [N, K/32].  bias f32 [N].
 * out: act_dtype for STORE / GELU, f32 for RESID; row pitch ldo >= N.
 * K % (128 / element size) == 0, N % 64 == 0. */
jepa_status jepa_op_gemm(int act_dtype, const void *a, int64_t M, int64_t K, const void *w,
                         int w_dtype, const uint16_t *w_scale, int64_t N, const float *bias,
                         int epilogue, void *out, int64_t ldo, void *hip_stream);

/* The qkv linear layer (attn_qkv, Quantization page "The rule") with V
 * written transposed for attention: acc = a[M, K] * w[N, K]^T + bias in
 * f32, N = 3*heads*64, weights as in jepa_op_gemm.  Columns [0, 2*heads*64)
 * (q and k) -> qk_out act [M, ld_qk] (ld_qk >= N; columns N - heads*64 .. N-1
 * of qk_out are not written); columns [2*heads*64, N) (v) -> vt act
 * [M / n_tokens, heads, 64, npad], row b*n_tokens + n being token n of item
 * b, each value rounded once to the act dtype.  Within a vt row, token n is
 * at position JEPA_VT_POS(n): each aligned run of 16 tokens is stored in the
 * order 0-3, 8-11, 4-7, 12-15, the order the attention kernel's operands
 * read.  Positions holding no token are not written.  rope (NULL: none),
 * f32 device [n_tokens, 32, 2] as jepa_rope_table writes it: q and k of
 * token n (row b*n_tokens + n), dims (2p, 2p+1) of every head, are rotated
 * by the angle whose (cos, sin) is entry (n, p), in f32, before the scale.
 * q_scale (0 or 1: none) then multiplies the q columns before their
 * rounding, e.g. JEPA_ATTN_Q_SCALE for jepa_op_attention's q_prescaled.
 * M % n_tokens == 0, npad >= n_tokens rounded up to 16. */
jepa_status jepa_op_gemm_qkv(int act_dtype, const void *a, int64_t M, int64_t K, const void *w,
                             int w_dtype, const uint16_t *w_scale, int heads, const float *bias,
                             int n_tokens, void *qk_out, int64_t ld_qk, void *vt, int64_t npad,
                             const float *rope, float q_scale, void *hip_stream);

/* The v columns of a qkv matrix act [batch*n_tokens, 3*heads*64] transposed
 * per head into vt act [batch, heads, 64, npad], token n at position
 * JEPA_VT_POS(n) of its row (positions holding no token not written). */
jepa_status jepa_op_transpose_v(int act_dtype, const void *qkv, int batch, int n_tokens,
                                int heads, void *vt, int64_t npad, void *hip_stream);

/* Multi-head attention, head_dim 64 (LeVJEPA card, opening paragraph, for
 * the block-causal mask).  q and k: act rows of pitch ld_qk elements (token
 * item*n_tokens + n), q of head h at column h*64, k at column heads*64 +
 * h*64; v: vt act [batch, heads, 64, npad] as written by jepa_op_transpose_v
 * (token n at JEPA_VT_POS(n)), npad = n_tokens rounded up to 64, positions
 * holding no token finite (zero).
 * -> out act [batch*n_tokens, heads*64].  mask JEPA_MASK_BLOCK_CAUSAL groups
 * the patch tokens (after the optional CLS token 0) in consecutive runs of
 * tokens_per_slot.  q_prescaled: the q columns hold q * JEPA_ATTN_Q_SCALE
 * (as jepa_op_gemm_qkv writes them with that q_scale), so q.k is already the
 * base-2 softmax exponent; otherwise q is the plain projection. */
jepa_status jepa_op_attention(int act_dtype, const void *qk, int64_t ld_qk, const void *vt,
                              int64_t npad, int batch, int n_tokens, int heads, int has_cls,
                              int mask, int tokens_per_slot, int q_prescaled, void *out,
                              void *hip_stream);

/* Host: the table of 3-D rotary position (see jepa_dims.rope; V-JEPA 2
 * card, opening paragraph) for the token grid of dims: out f32 host
 * [N, 32, 2], N = tokens per item, entry (n, p) = (cos, sin) of the angle of
 * token n's dimension pair p: for a patch token at (slot t, row h, column w),
 * pair 10a + i (a < 3, i < 10) has angle (t, h, w)[a] * 10000^(-i/10);
 * pairs 30 and 31, and every pair of a CLS token, have angle 0.  Angles and
 * their cos / sin are evaluated in double and rounded once to f32.  dims is
 * validated as by jepa_create (rope itself may be 0 or 1). */
jepa_status jepa_rope_table(const jepa_dims *dims, float *out);

/* Host: split Q8_0 / Q4_0 blocks [rows, cols/32] into the device layout
 * the GEMM reads: codes (rows*cols bytes of int8 for Q8_0; rows*cols/2
 * bytes of 16-byte nibble blocks for Q4_0) and scales (rows*cols/32 f16).
 * A copy only: no value changes. */
jepa_status jepa_pack_blocks(int dtype, const uint8_t *blocks, int64_t rows, int64_t cols,
                             uint8_t *codes, uint16_t *scales);

#ifdef __cplusplus
}
#endif

#endif /* JEPA_MI355X_OPS_H */
