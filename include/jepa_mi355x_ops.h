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

/* log2(e) / sqrt(head_dim) for head_dim 64 and 32.  q multiplied by it
 * turns q.k into the base-2 exponent of the softmax (scale 1/sqrt(head_dim),
 * base e); jepa_encode folds it into the qkv layer's q columns (q_scale) and
 * runs attention with q_prescaled. */
#define JEPA_ATTN_Q_SCALE 0.18033688011112042f
#define JEPA_ATTN_Q_SCALE_32 0.25503486164919736f

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

/* Patch embedding straight from the frames (the encoder's front end: LeVJEPA
 * card and V-JEPA 2 card, opening paragraphs: tubelet 1 or 2, patch 16):
 * out[b, has_cls + n, :] = W * x + bias (+ pos[has_cls + n, :]) for patch n
 * of item b, where x is its patch vector (dt, dy, dx, c; c fastest) of the
 * normalised pixels u * (1 / (255 std_c)) + (-mean_c / std_c) (constants
 * rounded once from double to f32), rounded to act_dtype; the f32 product
 * sums in f32.  The GEMM gathers x from the frames as it loads its tiles;
 * no patch matrix is written.  frames: device uint8 [B, T, H, W, 3],
 * 8-byte aligned; (patch * 3) % 8 == 0 and (W * 3) % 8 == 0.  w: act_dtype
 * [n, k_pitch], k_pitch >= tubelet * patch^2 * 3 a multiple of 64 up to
 * 2048 (columns past the patch length are never read as data: the gathered
 * values there are 0).  bias f32 [n], pos f32 [N_tok, n] or NULL, out f32
 * [B, N_tok, n] with N_tok = patches + has_cls; CLS rows are not written.
 * n % 64 == 0.  JEPA_E_HIP (invalid value) for shapes outside these. */
jepa_status jepa_op_patch_embed(int act_dtype, const uint8_t *frames, int B, int T, int H, int W, int tubelet,
                                int patch, const float *mean, const float *std, const void *w, int64_t k_pitch,
                                int64_t n, const float *bias, const float *pos, int has_cls, float *out,
                                void *hip_stream);

/* Activations quantised per 32-block for the int8 path (see
 * jepa_set_int8_matmul): x act_dtype (F16 / BF16) [rows, k], k % 32 == 0,
 * 16-byte aligned -> codes_out int8 [rows, k] (16-byte aligned) and
 * scales_out f32 [rows, k / 32]: for each block of 32 values of a row,
 * d = max|x| / 127 and code = round(x / d) half away from zero (0 when d is
 * 0), both in f32. */
jepa_status jepa_op_quantize_act(int act_dtype, const void *x, int64_t rows, int64_t k, int8_t *codes_out,
                                 float *scales_out, void *hip_stream);

/* The int8 product of jepa_set_int8_matmul: acc[m, n] = bias[n] + sum over
 * the K / 32 blocks b of a_scales[m, b] * d_w[n, b] * (the int32 dot product
 * of a_codes[m, block b] and the weight codes of row n, block b), in f32,
 * then jepa_op_gemm's epilogue into out (act_dtype F16 / BF16 for STORE /
 * GELU, f32 for RESID; pitch ldo >= N).  a_codes int8 [M, K], a_scales f32
 * [M, K / 32] as jepa_op_quantize_act writes them; w packed Q8_0 (codes
 * int8) or Q4_0 (codes nibble - 8) as for jepa_op_gemm, w_scale their f16
 * scales [N, K / 32].  K % 128 == 0, N % 64 == 0; a_codes and w 16-byte
 * aligned, a_scales 8-byte, w_scale 4-byte, bias and out 16-byte.
 * JEPA_E_HIP (invalid value) for shapes or alignments outside these. */
jepa_status jepa_op_gemm_i8(int act_dtype, const int8_t *a_codes, const float *a_scales, int64_t M, int64_t K,
                            const void *w, int w_dtype, const uint16_t *w_scale, int64_t N, const float *bias,
                            int epilogue, void *out, int64_t ldo, void *hip_stream);

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
 * f32, D = heads*head_dim (head_dim 32 or 64), N = 3*D, weights as in
 * jepa_op_gemm.  Columns [0, 2D) (q and k) -> qk_out act [M, ld_qk]
 * (ld_qk >= N; columns 2D .. N-1 of qk_out are not written); columns
 * [2D, N) (v) -> vt act [M / n_tokens, D, npad]: row b*D + c of vt holds v
 * column c (head c / head_dim, dim c % head_dim) of item b's tokens, row
 * b*n_tokens + n of a being token n of item b, each value rounded once to
 * the act dtype.  Within a vt row, token n is at position JEPA_VT_POS(n):
 * each aligned run of 16 tokens is stored in the order 0-3, 8-11, 4-7,
 * 12-15, the order the attention kernel's operands read.  Positions holding
 * no token are not written.  rope (NULL: none), f32 device
 * [n_tokens, head_dim/2, 2] as jepa_rope_table writes it: q and k of token
 * n, dims (2p, 2p+1) of every head, are rotated by the angle whose
 * (cos, sin) is entry (n, p), in f32, before the scale.  q_scale (0 or 1:
 * none) then multiplies the q columns before their rounding, e.g.
 * JEPA_ATTN_Q_SCALE(_32) for jepa_op_attention's q_prescaled.
 * M % n_tokens == 0, npad >= n_tokens rounded up to 16. */
jepa_status jepa_op_gemm_qkv(int act_dtype, const void *a, int64_t M, int64_t K, const void *w,
                             int w_dtype, const uint16_t *w_scale, int heads, int head_dim,
                             const float *bias, int n_tokens, void *qk_out, int64_t ld_qk, void *vt,
                             int64_t npad, const float *rope, float q_scale, void *hip_stream);

/* The v columns of a qkv matrix act [batch*n_tokens, 3*D], D =
 * heads*head_dim, transposed into vt act [batch, D, npad] (the layout
 * jepa_op_gemm_qkv writes), token n at position JEPA_VT_POS(n) of its row
 * (positions holding no token not written). */
jepa_status jepa_op_transpose_v(int act_dtype, const void *qkv, int batch, int n_tokens,
                                int heads, int head_dim, void *vt, int64_t npad, void *hip_stream);

/* Multi-head attention, head_dim 64 or 32 (LeVJEPA card, opening paragraph,
 * for the block-causal mask; head_dim 32 is the V-JEPA 2 predictor's width).
 * q and k: act rows of pitch ld_qk elements (token item*n_tokens + n), q of
 * head h at column h*head_dim, k at column D + h*head_dim, D =
 * heads*head_dim; v: vt act [batch, D, npad] as written by
 * jepa_op_transpose_v (token n at JEPA_VT_POS(n)), npad = n_tokens rounded
 * up to 64, positions holding no token finite (zero).
 * -> out act [batch*n_tokens, D].  mask JEPA_MASK_BLOCK_CAUSAL groups the
 * patch tokens (after the optional CLS token 0) in consecutive runs of
 * tokens_per_slot.  q_prescaled: the q columns hold q * log2(e) /
 * sqrt(head_dim) (JEPA_ATTN_Q_SCALE or _32, as jepa_op_gemm_qkv writes them
 * with that q_scale), so q.k is already the base-2 softmax exponent;
 * otherwise q is the plain projection. */
jepa_status jepa_op_attention(int act_dtype, const void *qk, int64_t ld_qk, const void *vt,
                              int64_t npad, int batch, int n_tokens, int heads, int head_dim,
                              int has_cls, int mask, int tokens_per_slot, int q_prescaled,
                              void *out, void *hip_stream);

/* Host: the table of 3-D rotary position (see jepa_dims.rope; V-JEPA 2
 * card, opening paragraph) for the token grid of dims: out f32 host
 * [N, dh/2, 2], N = tokens per item, dh = dim/heads, entry (n, p) =
 * (cos, sin) of the angle of token n's dimension pair p.  With ds =
 * 2*floor(dh/6) (20 for dh 64, 10 for 32), a patch token at (slot t, row h,
 * column w) has, for pair a*ds/2 + i (a < 3, i < ds/2), the angle
 * (t, h, w)[a] * 10000^(-2i/ds); the remaining pairs, and every pair of a
 * CLS token, have angle 0.  Angles and their cos / sin are evaluated in
 * double and rounded once to f32.  dims is validated as by jepa_create
 * (rope itself may be 0 or 1). */
jepa_status jepa_rope_table(const jepa_dims *dims, float *out);

/* Calibration of the dense bf16 MFMA rate (not part of the encoder): each of
 * `workgroups` workgroups of 4 waves runs iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands and writes one float
 * per thread to out (device f32, workgroups * 256 elements).  Work per launch:
 * workgroups * 4 * iters * 8 * 32768 flops; the caller times the launch.
 * operands: 0 = small constant values, the same bits in every instruction;
 * 1 = random values in [-1, 1), consecutive instructions differing in both
 * operands as in a GEMM (the matrix core's power, hence the clock the chip
 * sustains, grows with the operand bits that toggle).  Other values:
 * JEPA_E_INVALID_ARG. */
jepa_status jepa_op_mfma_probe(int workgroups, int iters, int operands, float *out, void *hip_stream);

/* The int8 MFMA rate, and what consuming it costs when every 32-wide K block
 * carries its own scales (the q8_0 weight format of the jepa.cpp
 * Quantization page, "The rule"; the int8 matrix path the Benchmarks page's
 * "Effect of the weight dtype" GPU table measures).  Each of `workgroups`
 * workgroups of 4 waves runs iters x 4 independent v_mfma_i32_32x32x32_i8
 * (65536 ops each) on register operands.  mode 0: products accumulate in
 * int32.  mode 1: each block's int32 result starts from zero and is added
 * into f32 accumulators scaled by a per-block scale of each of the lane's
 * rows times one of its column (convert, multiply, fused multiply-add per
 * element; scales read from LDS).  mode 2: as 1 with a single scale per
 * row for all of K (convert, fused multiply-add).  out: device f32,
 * workgroups * 256 elements (one sum per thread).  Ops per launch:
 * workgroups * 4 * iters * 4 * 65536; the caller times the launch. */
jepa_status jepa_op_mfma_i8_probe(int workgroups, int iters, int mode, float *out, void *hip_stream);

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
