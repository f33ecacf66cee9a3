// Host-side launchers of the gfx950 kernels.  Every launcher checks that the
// shapes fit what its kernel and grid assume and returns hipErrorInvalidValue
// otherwise; it never launches an out-of-contract grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jepa {

// ---- patchify: uint8 frames -> normalised patch matrix ---------------------
struct PatchifyArgs {
    const uint8_t *frames;   // [B, T, H, W, 3]
    int B, T, H, W, tubelet, patch;
    float mean[3], std[3];
    void *out;               // act dtype [B*Np, ld]; columns >= P are zero
    int64_t ld;              // row pitch in elements (>= P, multiple of 64)
};
hipError_t launch_patchify(int act_dt, const PatchifyArgs &a, hipStream_t s);

// ---- LayerNorm: f32 rows -> y in f32 / f16 / bf16 ----------------------------
hipError_t launch_layernorm(const float *x, int64_t rows, int dim, const float *gamma,
                            const float *beta, float eps, void *y, int y_dt, hipStream_t s);

// ---- GEMM: out = epilogue(A[M, K] * W[N, K]^T + bias) -----------------------
enum Epi { EPI_STORE = 0, EPI_GELU = 1, EPI_RESID = 2, EPI_PATCH = 3, EPI_QKV = 4 };
struct GemmArgs {
    const void *a;           // act dtype [M, K] row-major, pitch lda elements
    const void *w;           // dense: act dtype [N, K]; q8_0: int8 codes [N, K];
                             // q4_0: nibble blocks [N, K/2]
    const uint16_t *wscale;  // q formats: f16 scales [N, K/32]
    const float *bias;       // [N]
    void *out;               // STORE/GELU: act dtype [M, ldo]; RESID/PATCH: f32
    int64_t M, N, K, lda, ldo;
    // EPI_PATCH: row r = b*np + n goes to output row b*ntok + has_cls + n and
    // adds pos[has_cls + n] (pos null: nothing)
    const float *pos;
    int np, ntok, has_cls;
    // EPI_QKV: columns < vcol0 as EPI_STORE; columns >= vcol0 (the v part,
    // heads of 64) go transposed to vt [M / ntok, (N - vcol0) / 64, 64, npad],
    // row r = b*ntok + n being token n of item b
    void *vt;
    int64_t npad, vcol0;
    // EPI_QKV: with rope (else null), f32 [ntok, head_dim / 2] (cos, sin)
    // pairs, the q and k columns' dims (2p, 2p+1) of each head of token
    // n = row % ntok are rotated by entry (n, p) first; then the q columns
    // [0, vcol0 / 2) are multiplied by qscale before rounding (0: left as
    // they are)
    const float *rope;
    int head_dim;            // 32 or 64 (the rotary pairs' period)
    float qscale;
    // EPI_QKV: set by the launcher when every item starts its tokens at a
    // multiple of 16 rows (ntok % 16 == 0, or one item): the large tile
    // then writes V^T straight from its accumulators
    int vt_direct;
    // launches of this shape expected to run concurrently (batch parts on
    // other streams; 0 or 1: none), a hint for the tile-shape choice
    int conc;
    // first row of this launch: a launch covers rows [m_begin, M), all row
    // indices above stay absolute (set by the launcher when it gives a
    // GEMM's last rows their own, smaller tiles; callers pass 0)
    int64_t m_begin;
    // f32 EPI_RESID with few tiles: scratch for a K split (KSPLIT_MAX * M * N
    // floats, or null: no split); each split's partial product goes there and
    // a second pass adds the bias and the splits in order to the output
    float *kpart;
    int ksplit;              // set by the launcher
    // int8 path (launch_gemm_i8): a holds int8 codes [M, lda] (lda bytes),
    // ascale their f32 scales [M, K/32], one per 32-block of a row
    const float *ascale;
    // EPI_PATCH straight from the frames (implicit GEMM; a unused): uint8
    // [items, fT, fH, fW, 3], row r = b*np + n being patch n of item b, its
    // patch vector (dt, dy, dx, c) gathered and normalised on the way into
    // LDS as act(u * pix_scale[c] + pix_shift[c]); K columns >= patch_len
    // read as 0.  Needs a 16-bit act dtype, (patch * 3) % 8 == 0,
    // (fW * 3) % 8 == 0 and 8-byte aligned frames.
    const uint8_t *frames;
    int fT, fH, fW, tubelet, patch, patch_len;
    float pix_scale[3], pix_shift[3];
};
constexpr int KSPLIT_MAX = 8;
hipError_t launch_gemm(int act_dt, int w_dt, int epi, const GemmArgs &g, hipStream_t s);
// The int8 path of q8_0 / q4_0 matrices: g.a / g.ascale hold activations
// quantised per 32-block (launch_quant_act), the products of every block
// run on int8 MFMA and are scaled by d_a * d_w into f32 accumulators; the
// epilogues (STORE, GELU, RESID, QKV) and out act_dt (16-bit) are
// launch_gemm's.  K a multiple of 128, N of 64.
hipError_t launch_gemm_i8(int act_dt, int w_dt, int epi, const GemmArgs &g, hipStream_t s);
// x act [M, ldx] (16-bit) -> codes int8 [M, ldq] and f32 scales [M, K/32]
// (pitch K/32): per 32-block of a row d = max|x| / 127 and code
// round(x / d) half away from zero (0 when d is 0), both in f32
hipError_t launch_quant_act(int act_dt, const void *x, int64_t ldx, int64_t M, int64_t K, int8_t *q,
                            int64_t ldq, float *d, hipStream_t s);

// Position of token n in a V^T row: each aligned run of 16 tokens is stored
// in the order 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 swapped), so the eight
// keys one lane of the PV MFMA operand needs are 16 contiguous bytes.
__host__ __device__ __forceinline__ int64_t vt_pos(int64_t n) {
    return (n & ~(int64_t)12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

// ---- attention --------------------------------------------------------------
// Q and K: act dtype rows of pitch ld_qk, q of head h at column h*dh, k at
// column D + h*dh.  V transposed: vt [B, D, npad] (head h's dims at rows
// h*dh..), npad = N rounded up to 64, columns N..npad-1 finite (zero).
struct AttnArgs {
    const void *qk;
    int64_t ld_qk;
    const void *vt;
    int64_t npad;
    void *out;               // act dtype [B*N, D]
    int B, N, heads, has_cls, block_causal, per_slot;
    int q_prescaled;         // q already multiplied by ATTN_Q_SCALE
    int dh;                  // head dim: 32 or 64
    // f32 path with few workgroups: scratch for a key split (KVSPLIT_MAX *
    // B * heads * N * (dh + 2) floats, or null: no split); each split's
    // unnormalised output, max and sum go there and a second pass merges them
    float *kvpart;
    int kvsplit;             // set by the launcher
};
// log2(e) / sqrt(64): with q multiplied by it, q.k is the exponent of the
// softmax in base 2 (head dim 64; for head dim 32, log2(e) / sqrt(32))
constexpr float ATTN_Q_SCALE = 0.18033688011112042f;
constexpr int KVSPLIT_MAX = 8;
constexpr float ATTN_Q_SCALE_32 = 0.25503486164919736f;
__host__ __device__ constexpr float attn_q_scale(int dh) { return dh == 32 ? ATTN_Q_SCALE_32 : ATTN_Q_SCALE; }
hipError_t launch_attention(int act_dt, const AttnArgs &a, hipStream_t s);
// vt [B, D, npad] <- the v columns of a [B*N, 3D] qkv matrix, transposed
hipError_t launch_transpose_v(int act_dt, const void *qkv, int B, int N, int D, void *vt,
                              int64_t npad, hipStream_t s);

// One query row per item attending over that item's N key / value rows
// (the classifier head's cross-attention): q act [B, D], k and v act rows
// of pitch ldkv (token b*N + n), heads of dh (32 or 64), softmax scale
// 1/sqrt(dh) -> out act [B, D].  N <= XATTN_MAX_N.
constexpr int XATTN_MAX_N = 16384;
hipError_t launch_xattn(int act_dt, const void *q, const void *k, const void *v, int64_t ldkv, int B, int N,
                        int heads, int dh, void *out, hipStream_t s);

// ---- small helpers ----------------------------------------------------------
// y (act dtype) <- x (f32), n elements; x <- v, n elements
hipError_t launch_cast(const float *x, int64_t n, void *y, int y_dt, hipStream_t s);
hipError_t launch_fill(float *x, int64_t n, float v, hipStream_t s);
// dense bf16 MFMA calibration: workgroups x 4 waves, each iters x 8
// independent 32x32x16 MFMAs; out holds workgroups * 256 floats
hipError_t launch_mfma_probe(int workgroups, int iters, int operands, float *out, hipStream_t s);
// int8 MFMA calibration: mode 0 plain, 1 / 2 with per-block rescaling into
// f32 (see misc.hip); workgroups x 4 waves, each iters x 4 32x32x32 MFMAs
hipError_t launch_mfma_i8_probe(int workgroups, int iters, int mode, float *out, hipStream_t s);
// X[b*N + 0] = cls + pos[0] for every item (pos null: cls)
hipError_t launch_cls_rows(float *x, const float *cls, const float *pos, int B, int N, int D,
                           hipStream_t s);
// pooling of a token map y [B, N, D]
hipError_t launch_copy_f32(const float *y, int64_t n, float *out, hipStream_t s);
hipError_t launch_pool_cls(const float *y, int B, int N, int D, float *out, hipStream_t s);
// mean pool via per-chunk partial sums: part holds B * POOL_CHUNKS * D floats
constexpr int POOL_CHUNKS = 32;
hipError_t launch_pool_mean(const float *y, int B, int N, int D, int first, float *part, float *out,
                            hipStream_t s);
// Block-format matrices expanded to the activation dtype, act(w) with w the
// f32 value of each weight (for q8_0 / q4_0 f32(d) * q, the values the
// GEMM's own dequantising tile load makes).  Job j covers the matrix's units
// of 32 weights [blk0_j, blk0_{j+1}) of the concatenated range (blk0
// ascending, blk0_0 = 0); dst is the act-dtype matrix [rows, cols] (16-byte
// aligned).  Device layouts (each field as stored, split into arrays):
//   q8_0: codes int8 [units][32]; scale f16 [units]
//   q4_0: codes [units][16] (byte j: code j low nibble, code j+16 high);
//         scale f16 [units]
//   q4_K: codes [super-blocks][128] (the stored 4-bit codes); scale f16
//         [super-blocks][2] (d, dmin); sub [super-blocks][12] (the stored
//         6-bit sub-block scales and mins)
//   q6_K: codes [super-blocks][192] (the 128 low-bit then 64 high-bit
//         bytes); scale f16 [super-blocks] (d); sub int8 [super-blocks][16]
// (a super-block is 256 weights, 8 units, along a row)
struct ExpandJob {
    const void *codes;
    const uint16_t *scale;
    const uint8_t *sub;
    void *dst;
    int64_t blk0;
    int w_dt;
};
hipError_t launch_expand(int act_dt, const ExpandJob *jobs, int njobs, int64_t nblk, hipStream_t s);
// dequantise block formats (layouts as above), or widen f16 / bf16 / f32
// storage, into f32 [rows, cols]
hipError_t launch_dequant(int w_dt, const void *w, const uint16_t *scale, const uint8_t *sub, int64_t rows,
                          int64_t cols, float *out, hipStream_t s);

}  // namespace jepa
