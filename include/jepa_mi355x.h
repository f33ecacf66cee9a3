/*
 * jepa_mi355x.h -- C ABI of the MI355X (gfx950) JEPA ViT encoder forward pass.
 *
 * The operation: a clip of uint8 frames is normalised, cut into tubelet
 * patches, embedded, run through pre-LN transformer blocks with bidirectional
 * or block-causal multi-head attention, final-LayerNorm'ed into a token map,
 * and optionally pooled (CLS or mean).
 *   - LeVJEPA ViT-L/16 (VideoMix) model card, opening paragraph: tubelet 1;
 *     the mask that lets a patch token see the tokens of its own and earlier
 *     temporal slots but never the CLS token, while CLS sees every token;
 *     the CLS token as the feature; "Run it": the pooling modes and the
 *     single C header.
 *   - V-JEPA 2 ViT-L/16 SSv2 card, opening paragraph: tubelet 2.
 *   - jepa.cpp Quantization page, "The rule": the tensor names, which
 *     tensors may be stored as q8_0 / q4_0 / q4_K / q6_K blocks, and the
 *     K-quants' fallback for rows that are not a multiple of 256; "File
 *     sizes": 8.5 / 4.5 bits per weight; "CLI": q4_K block sizes.
 *   - jepa.cpp benchmarks page, "What the milliseconds are": the per-call
 *     compute time and the resident model bytes the API reports.
 *
 * Conventions shared by every call:
 *   - No call aborts, exits or throws.  Each returns a jepa_status; on a
 *     negative status jepa_last_error() names the field or tensor at fault.
 *     Arguments are validated before anything is enqueued.
 *   - Device work is enqueued on the caller's HIP stream (a hipStream_t
 *     passed as void*; NULL means the default stream) and the call returns
 *     after enqueueing, except where noted.  Outputs are valid once the
 *     caller synchronises that stream.  Device faults surface there.
 *   - One context must not be used from two threads at once.
 *   - A context's calls share its device workspace (staged frames, the
 *     residual stream, the token map, scratch).  Successive calls on one
 *     context must therefore be ordered on the GPU: issue them on one stream,
 *     or synchronise the earlier call's stream before issuing on another.
 *   - The library needs a gfx950 device; it has no CPU fallback.
 */
#ifndef JEPA_MI355X_H
#define JEPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct jepa_ctx jepa_ctx;

typedef enum {
    JEPA_OK = 0,
    JEPA_E_INVALID_ARG = -1,     /* null pointer, bad enum, batch <= 0 */
    JEPA_E_SHAPE = -2,           /* inconsistent dims or tensor shape */
    JEPA_E_DTYPE = -3,           /* dtype not allowed for this tensor */
    JEPA_E_MISSING_TENSOR = -4,  /* a required tensor is absent */
    JEPA_E_OOM = -5,             /* device allocation failed or over the cap */
    JEPA_E_HIP = -6,             /* a HIP runtime call or launch failed */
    JEPA_E_UNSUPPORTED = -7,     /* valid but outside what the library implements */
    JEPA_E_STATE = -8,           /* e.g. pool before any encode */
    JEPA_E_FORMAT = -9           /* a model file is malformed or lacks a required key */
} jepa_status;

/* Storage dtypes.  Q8_0: blocks of 32 weights along a row, each an f16
 * scale d then 32 int8 codes (34 bytes), weight = d * q.  Q4_0: blocks of
 * 32, an f16 scale d then 16 bytes whose byte j holds code j in the low
 * nibble and code j + 16 in the high nibble (18 bytes), weight = d*(q-8).
 * The K-quants (ggml's published layouts; 256 weights per super-block,
 * eight sub-blocks of 32):
 * Q4_K (144 bytes): f16 d, f16 dmin, 12 bytes of 6-bit sub-block scales
 *   sc_j and mins m_j (j < 4: sc_j = s[j] & 63, m_j = s[j+4] & 63; j >= 4:
 *   sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4, m_j = (s[j+4] >> 4) |
 *   (s[j] >> 6) << 4), then 128 code bytes: bytes 32p..32p+31 hold
 *   sub-block 2p in their low nibbles and 2p+1 in their high ones;
 *   weight = d sc_j q - dmin m_j.
 * Q6_K (210 bytes): 128 bytes of low 4 code bits, 64 bytes of high 2 bits,
 *   16 int8 scales (one per 16 weights), f16 d.  Weight 128h + 32t + l
 *   (h < 2, t < 4, l < 32) takes the low (t < 2) or high nibble of low byte
 *   64h + 32(t%2) + l and bits 2t, 2t+1 of high byte 32h + l;
 *   weight = d scale (q - 32). */
typedef enum { JEPA_F32 = 0, JEPA_F16 = 1, JEPA_BF16 = 2, JEPA_Q8_0 = 3, JEPA_Q4_0 = 4, JEPA_Q4_K = 5,
               JEPA_Q6_K = 6 } jepa_dtype;

typedef enum { JEPA_MASK_BIDIR = 0, JEPA_MASK_BLOCK_CAUSAL = 1 } jepa_mask;

typedef enum { JEPA_POOL_NONE = 0, JEPA_POOL_CLS = 1, JEPA_POOL_MEAN = 2 } jepa_pool_mode;

/* Model dimensions.  head_dim = dim / heads must be 64 or 32; dim and mlp_dim
 * must be multiples of 64; img_h, img_w divisible by patch; frames divisible
 * by tubelet.  Tokens per item: N = (frames/tubelet)*(img_h/patch)*(img_w/patch)
 * + has_cls.  Pixels are normalised as (u/255 - mean[c]) / std[c].
 * act_dtype (F32, F16 or BF16) is the precision of the GEMM and attention
 * operands; accumulation, the residual stream, LayerNorm statistics and
 * softmax are f32 throughout.  Under JEPA_MASK_BLOCK_CAUSAL a patch token of
 * temporal slot t attends to the patch tokens of slots <= t and not to CLS;
 * CLS attends to every token.
 * rope = 1 selects 3-D rotary position (V-JEPA 2 card, opening paragraph:
 * the encoder uses "3-D RoPE"; the rotation is RoFormer's) instead of the
 * additive table enc.pos_embed, which is then not part of the schema: in
 * every block, before the scores, each head's q and k are rotated pairwise,
 * dims (2i, 2i+1) of segment a (a = 0, 1, 2: temporal slot, patch row, patch
 * column, ds = 2*floor(head_dim/6) dims each: 20 of 64, 10 of 32; the dims
 * after the three segments untouched) by pos_a * 10000^(-2i/ds) radians.  A
 * CLS token has no position and is not rotated.
 * head_classes > 0 adds the attentive-pool classifier head (V-JEPA 2 SSv2
 * card, opening paragraph; benchmarks page, "Attentive-pool head"), run by
 * jepa_classify on the final token map: head_blocks pre-LN blocks as the
 * encoder's (bidirectional, no position terms) over every token; then one
 * learned query q0 attends, per head, over LN1(tokens) projected to keys and
 * values (the query is W_q q0 + b_q, with no LayerNorm); x = q0 +
 * out_proj(attention); x += MLP(LN2(x)) (erf GELU); scores = W_c x + b_c. */
typedef struct {
    int32_t dim, depth, heads, mlp_dim;
    int32_t patch, tubelet, img_h, img_w, frames;
    int32_t has_cls;    /* 1: token 0 of each item is a learned CLS token */
    int32_t mask;       /* jepa_mask */
    int32_t act_dtype;  /* jepa_dtype: JEPA_F32, JEPA_F16 or JEPA_BF16 */
    float ln_eps;
    float mean[3];
    float std[3];
    int32_t rope;       /* 0: additive enc.pos_embed; 1: 3-D rotary position */
    int32_t head_blocks;  /* classifier head: self-attention blocks (the V-JEPA 2 SSv2 head: 3) */
    int32_t head_classes; /* classifier head: classes (0 = no head; SSv2: 174) */
} jepa_dims;

/* One stored tensor, host memory.  ne0 = row length (in-features), ne1 =
 * rows (out-features; 1 for vectors).  nbytes must equal the storage size
 * of ne0*ne1 elements of dtype.  Names and shapes (D = dim, F = mlp_dim,
 * P = tubelet*patch*patch*3, N = tokens per item):
 *   enc.patch_embed.weight [ne0 P, ne1 D]   enc.patch_embed.bias [D]
 *   enc.cls_token [D] (only if has_cls)     enc.pos_embed [ne0 D, ne1 N] (not if rope)
 *   enc.blk.{i}.ln1.weight/.bias [D]        enc.blk.{i}.ln2.weight/.bias [D]
 *   enc.blk.{i}.attn_qkv.weight [D, 3D] .bias [3D]   (columns [q | k | v],
 *       head a owns features a*hd..a*hd+hd-1 of each third, hd = head_dim)
 *   enc.blk.{i}.attn_out.weight [D, D] .bias [D]
 *   enc.blk.{i}.ffn_up.weight [D, F] .bias [F]
 *   enc.blk.{i}.ffn_down.weight [F, D] .bias [D]
 *   enc.norm.weight/.bias [D]
 * With head_classes = C > 0, also (see jepa_dims):
 *   head.blk.{i}.* as enc.blk.{i}.*, for i < head_blocks
 *   head.query_token [D]   head.xattn.ln1/ln2.weight/.bias [D]
 *   head.xattn.attn_q/attn_k/attn_v/attn_out.weight [D, D] .bias [D]
 *   head.xattn.ffn_up.weight [D, F] .bias [F]   head.xattn.ffn_down.weight [F, D] .bias [D]
 *   head.classifier.weight [D, C] .bias [C]
 * A patch vector lists (dt, dy, dx, c) with c fastest; tokens are ordered
 * slot-major then raster; CLS is token 0 and owns pos row 0.
 * Only the attn_qkv / attn_q / attn_k / attn_v / attn_out / ffn_up /
 * ffn_down weights may take a block dtype (Q8_0 / Q4_0 with ne0 % 64 == 0,
 * Q4_K / Q6_K with ne0 % 256 == 0, else JEPA_E_SHAPE: a writer stores such
 * rows as Q4_0 / Q8_0 instead), and only with act_dtype F16 or BF16; the
 * rest are F32, F16 or BF16. */
typedef struct {
    const char *name;
    int32_t dtype;      /* jepa_dtype */
    int64_t ne0;
    int64_t ne1;
    const void *data;   /* host pointer */
    size_t nbytes;
} jepa_tensor;

/* ---- GGUF model files ----
 * The models travel as GGUF files that carry every dimension, the
 * positional scheme and the preprocessing recipe (LeVJEPA card, opening
 * paragraph), re-typed by the rule of the jepa.cpp Quantization page ("The
 * rule"), whose general.file_type names the requested type even where a
 * K-quant tensor fell back.
 * Container read: GGUF version 2 or 3, little-endian; general.alignment
 * (default 32).  Tensor types (ggml ids): f32 0, f16 1, q4_0 2, q8_0 8,
 * q4_K 12, q6_K 14, bf16 30; the other ggml types are reported by name as
 * JEPA_E_UNSUPPORTED.  A tensor's first dimension is its row length ne0,
 * the product of the others its ne1; names and shapes as in jepa_tensor.
 * Keys (this library's schema, the file's own model description):
 *   general.architecture  string "jepa" (required)
 *   jepa.dim, jepa.depth, jepa.heads, jepa.mlp_dim, jepa.patch, jepa.img_h,
 *   jepa.img_w, jepa.has_cls   integers (required)
 *   jepa.tubelet, jepa.frames  integers (default 1)
 *   jepa.rope, jepa.head.blocks, jepa.head.classes  integers (default 0)
 *   jepa.mask      string "bidirectional" (default) or "block_causal"
 *   jepa.ln_eps    number (default 1e-6)
 *   jepa.pre.mean, jepa.pre.std   arrays of 3 floats (required)
 *   general.file_type   integer (optional, reported)
 * Other keys are ignored.  Every offset and length is checked against the
 * file's size before use: a malformed file returns JEPA_E_FORMAT (or
 * JEPA_E_UNSUPPORTED for a valid file this library cannot run), never a
 * crash. */
typedef struct {
    jepa_dims dims;        /* from the keys; act_dtype = JEPA_F32 */
    int32_t version;
    int32_t file_type;     /* general.file_type, -1 when absent */
    int64_t n_tensors, n_kv;
    int64_t alignment;
    int64_t data_offset;   /* byte offset of the tensor data section */
    int64_t tensor_bytes;  /* sum of the tensors' storage sizes */
} jepa_gguf_info;

/* Read a GGUF file's header, keys and tensor records (host only; touches
 * no device). */
jepa_status jepa_gguf_read_info(const char *path, jepa_gguf_info *info);

/* jepa_create from a GGUF file, its tensors read from a read-only mapping
 * of the file (unmapped before return).  act_dtype: JEPA_F32, JEPA_F16 or
 * JEPA_BF16, or -1 for F32 when every tensor is f32, BF16 when the others
 * are bf16, else F16. */
jepa_status jepa_create_from_gguf(const char *path, int act_dtype, jepa_ctx **out);

/* The type a general.file_type code names ("f32", "f16", "q4_0", "q4_1",
 * "q8_0", "q5_0", "q5_1", "q4_k", "q5_k", "q6_k": the codes 0, 1, 2, 3, 7,
 * 8, 9, 12, 13, 14 of the Quantization page, "The rule"), or NULL. */
const char *jepa_file_type_name(int code);

/* Per-kernel-class timing record (see jepa_set_profiling). */
typedef struct {
    const char *name;   /* static string owned by the library */
    int64_t launches;
    double total_ms;
} jepa_kernel_stat;

/* Validate dims and tensors, allocate device memory on the current device,
 * copy every tensor there (the caller may free its buffers on return) and
 * return a context in *out.  Blocks until the copies are done.  Every name
 * in the schema above must be present exactly once; unknown names are an
 * error (JEPA_E_INVALID_ARG). */
jepa_status jepa_create(const jepa_dims *dims, const jepa_tensor *tensors, int n_tensors,
                        jepa_ctx **out);

/* Encode a batch.  frames: uint8 [batch, frames, img_h, img_w, 3], HWC,
 * contiguous; device memory if frames_on_device, else host memory, which is
 * copied into a context-owned pinned buffer before the call returns (the
 * caller may reuse it at once) and sent to the device on hip_stream.  tokens_out: device f32
 * [batch, N, dim] that receives the final-LayerNorm token map, or NULL to
 * keep it in a context-owned buffer.  jepa_pool and jepa_classify read the
 * token map where this call wrote it, so a caller-given tokens_out must stay
 * allocated (and unmodified) until the next encode on this context; they
 * write as many rows as this call's batch.  From the moment an encode is
 * called, the previous token map is forgotten: if the call fails, pool and
 * classify return JEPA_E_STATE until an encode succeeds. */
jepa_status jepa_encode(jepa_ctx *ctx, const uint8_t *frames, int batch, int frames_on_device,
                        float *tokens_out, void *hip_stream);

/* Size in bytes of the static device array jepa_encode_noalloc works in. */
#define JEPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* jepa_encode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It runs jepa_encode's launch sequence with the batch as one part, and its
 * buffers (residual stream, activations, V^T, split partial sums) live in
 * one static device array of JEPA_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds, at its own address, until the process ends.  No
 * hipMalloc, hipFree or other allocating call is made, and no timing events
 * are recorded.  frames: device uint8 [batch, frames, img_h, img_w, 3];
 * tokens_out: device f32 [batch, N, dim], required.  Q8_0 / Q4_0 matrices
 * are dequantised in the GEMM's tile load (no expanded copy); a model with
 * Q4_K / Q6_K matrices, which run from an expanded copy, is refused with
 * JEPA_E_UNSUPPORTED.  A batch whose
 * buffers do not fit the array is refused with JEPA_E_OOM before anything
 * is enqueued: it serves small models (ViT-Ti/14 f32 needs about 6 MB per
 * image), not the ViT-L video batches, which need jepa_encode.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the call clears what must start at zero itself): calls that
 * overlap on one GPU, from any stream, thread or context, race and corrupt
 * each other's results; order them on one stream.  Like jepa_encode it
 * forgets the context's previous token map: jepa_pool and jepa_classify
 * return JEPA_E_STATE and jepa_last_compute_ms -1 until the next
 * jepa_encode. */
jepa_status jepa_encode_noalloc(jepa_ctx *ctx, const uint8_t *frames, int batch, float *tokens_out,
                                void *hip_stream);

/* Concurrency of jepa_encode: the batch is split into `parts` contiguous
 * groups of items, encoded concurrently on the caller's stream and parts-1
 * internal non-blocking HIP streams (default priority) forked from and
 * joined back onto the caller's stream, so that the work still starts and
 * ends in the caller's stream order.  Items never interact, so the
 * result does not depend on parts; only the overlap of kernels does (one
 * part's last, partial round of workgroups runs beside another part's
 * kernels).  parts = 0 restores the default (4, or the JEPA_STREAMS
 * environment variable); the effective count is min(parts, batch).
 * JEPA_E_INVALID_ARG unless 0 <= parts <= 4. */
jepa_status jepa_set_batch_parts(jepa_ctx *ctx, int parts);

/* The int8 path of q8_0 / q4_0 matrices (Benchmarks page, "Effect of the
 * weight dtype on a GPU (encoder)": the quantised encoders' products run on
 * integer arithmetic; Quantization page: the q8_0 path quantises the
 * activations of every product).  With enable = 1, each of a block's four
 * products whose matrix is Q8_0 or Q4_0 first quantises its input per
 * 32-block along K (d = max|x| / 127 in f32, codes round(x / d) half away
 * from zero), then runs every block's integer dot product on int8 MFMA and
 * adds d_a * d_w * dot into f32 accumulators; the epilogues are unchanged.
 * The result differs from the default path by the activations'
 * quantisation (up to half a step per value).  enable = 0 restores the
 * default (act-dtype MFMA on dequantised weights).  Changing it frees the
 * workspace (after a device synchronisation); the next encode allocates
 * one with room for the quantised inputs.  The classifier head's blocks
 * follow it; its other products do not.  JEPA_E_UNSUPPORTED for f32
 * models, models with K-quant matrices, or dim / mlp_dim not multiples of
 * 128; JEPA_E_INVALID_ARG unless enable is 0 or 1. */
jepa_status jepa_set_int8_matmul(jepa_ctx *ctx, int enable);

/* Pool the token map of the last encode.  out: device f32 [batch, dim] for
 * CLS (token 0; needs has_cls) and MEAN (mean of the patch tokens, CLS
 * excluded), [batch, N, dim] for NONE (a copy of the token map).
 * JEPA_E_STATE if nothing was encoded yet. */
jepa_status jepa_pool(jepa_ctx *ctx, int mode, float *out, void *hip_stream);

/* Release everything the context owns.  NULL is ignored. */
void jepa_free(jepa_ctx *ctx);

/* Message for the last failing call on this thread ("" if none). */
const char *jepa_last_error(void);

/* Device milliseconds between the start and the end of the last encode
 * (HIP events on the encode's stream); waits for that encode to finish.
 * Negative if there was none. */
float jepa_last_compute_ms(jepa_ctx *ctx);

/* Class scores of the attentive-pool head for the token map of the last
 * jepa_encode on this context: logits_out device f32 [batch, head_classes].
 * JEPA_E_STATE before any encode, JEPA_E_UNSUPPORTED for a model without
 * a head.  Work is enqueued on hip_stream; the head's blocks reuse the
 * encode workspace, so the next encode must not start before it ends
 * (true on one stream). */
jepa_status jepa_classify(jepa_ctx *ctx, float *logits_out, void *hip_stream);

/* Bytes of tensor data as stored (the size the weight file's tensors would
 * take: 34 / 18 bytes per 32 weights for Q8_0 / Q4_0, 144 / 210 per 256 for
 * Q4_K / Q6_K, 2 or 4 bytes per element otherwise). */
size_t jepa_model_n_bytes(const jepa_ctx *ctx);

/* Bytes of device memory the context holds for weights. */
size_t jepa_device_weight_bytes(const jepa_ctx *ctx);

/* Bytes of device workspace an encode of `batch` items needs (with the
 * current batch-part setting).  It includes, for a model with block
 * matrices and batch parts of 1024 or more token rows, an activation-dtype
 * copy of those matrices (the GEMMs then run dense): the first such encode
 * allocates it and writes it from the blocks before its first layer, later
 * encodes reuse it (on any stream: they wait for that write), and it is
 * held until jepa_free; smaller batches dequantise inside the GEMM and need
 * no copy.  The environment variable
 * JEPA_Q_EXPAND = 0 or 1 forces either way, except that a model with a
 * Q4_K / Q6_K matrix always takes the copy.  With the int8 path on
 * (jepa_set_int8_matmul) no copy is made, and the workspace holds the
 * quantised inputs instead: 1 + 4/32 bytes per value of a
 * [batch * tokens, max(dim, mlp_dim)] matrix. */
size_t jepa_workspace_bytes(const jepa_ctx *ctx, int batch);

/* Write the f32 value of every element of the named tensor, as the GEMMs
 * see it before rounding to act_dtype, into device memory out_dev
 * ([ne1, ne0] row-major).  For Q8_0/Q4_0 this is f32(d) * code, exact; for
 * Q6_K d * scale * (q - 32), exact; for Q4_K the exact d sc q - dmin m
 * rounded once to f32. */
jepa_status jepa_dequant_tensor(jepa_ctx *ctx, const char *name, float *out_dev, void *hip_stream);

/* Host quantizer: f32 [rows, cols] -> Q8_0 or Q4_0 blocks [rows, cols/32]
 * (dst holds rows*cols/32*34 or *18 bytes).  Scale d computed in f32 and
 * stored as f16 (round to nearest even); Q8_0: d = max|x|/127, codes
 * round-half-away(x * (1/d)); Q4_0: d = m / -8 with m the first element of
 * largest magnitude, codes min(15, floor(x * (1/d) + 8.5)); zero blocks get
 * d = 0.  cols % 32 == 0. */
jepa_status jepa_quantize(int dtype, const float *src, int64_t rows, int64_t cols, uint8_t *dst);

/* Kernel timing: every launch whose class bit is set in class_mask (bit i
 * = record i of jepa_kernel_stats; 0 = off, 0xffffffff = all) is bracketed
 * by HIP events on its stream.  jepa_kernel_stats waits for the recorded
 * launches, adds them into per-class totals and copies up to `cap` records
 * into out; it returns the number of classes (or a negative status).
 * jepa_reset_kernel_stats clears the totals. */
jepa_status jepa_set_profiling(jepa_ctx *ctx, uint32_t class_mask);
int jepa_kernel_stats(jepa_ctx *ctx, jepa_kernel_stat *out, int cap);
void jepa_reset_kernel_stats(jepa_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* JEPA_MI355X_H */
