// NT GEMM on MFMA for the encoder's linear layers (qkv, out-proj, fc1, fc2,
// patch-embed): out = epilogue(A[M, K] * W[N, K]^T + bias), f32 accumulate.
//
// Tile: 128 x 128 outputs per workgroup of 4 waves (2 x 2, 64 x 64 each, as
// 2 x 2 blocks of 32 x 32 MFMA accumulators), K step = 128 bytes of each
// row (64 elements of a 16-bit type, 32 of f32).  A and W tiles are staged
// through LDS, double buffered, with the next step's global loads held in
// registers while the current step's MFMAs run.  Rows of LDS are padded by
// 16 bytes so that the 32 rows one MFMA operand read touches fall in
// distinct banks.
//
// Weight formats (jepa.cpp Quantization page, "The rule" and "File
// sizes"): dense in the activation dtype, or q8_0 / q4_0 blocks of 32 along
// each row, dequantised on the way into LDS as act(f32(d) * q).
//
// Epilogues, fused so that no separate elementwise pass touches HBM:
//   STORE  out = act(acc + b)                    (qkv)
//   GELU   out = act(gelu_erf(acc + b))          (fc1)
//   RESID  X  += acc + b   (f32 residual)        (out-proj, fc2)
//   PATCH  X[token] = acc + b + pos[token]       (patch-embed, CLS offset)
//   QKV    q, k columns as STORE (q optionally scaled first); v columns
//          transposed per head into V^T
#include <stdlib.h>
#include <string.h>

#include <string>
#include <type_traits>
#include <utility>

#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace jepa {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 144;                 // LDS bytes per tile row (128 + pad)
constexpr int TILEB = 128 * ROWB;         // LDS bytes per 128-row tile

// GELU, erf form: 0.5 z (1 + erf(z / sqrt 2)) = z Phi(z).  The f32 path
// keeps the library erf.  For 16-bit outputs it is written as
//   GELU(z) = max(z, 0) - |z| erfc(|z| / sqrt 2) / 2,
// the same function without the cancellation in 1 + erf for z < 0, with
// erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x) from Abramowitz & Stegun, Handbook of Mathematical
// Functions, 7.1.26 (Hastings): |error| <= 1.5e-7 for x >= 0.  One
// reciprocal, one exponential and nine other operations per value (the last
// an FMA onto max(z, 0)).
__device__ __forceinline__ float gelu_as7126(float z) {
    constexpr float P = 0.3275911f * 0.70710678118654752f;   // p / sqrt 2: t in terms of |z|
    const float t = __builtin_amdgcn_rcpf(fmaf(P, fabsf(z), 1.0f));
    float q = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);   // coefficients halved
    q = fmaf(q, t, 0.5f * 1.421413741f);
    q = fmaf(q, t, 0.5f * -0.284496736f);
    q = fmaf(q, t, 0.5f * 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(z * z * (-0.5f * 1.4426950408889634f));   // exp(-z^2 / 2)
    const float u = q * (t * e);                                                   // erfc(|z|/sqrt2) / 2
    // max(z, 0) - |z| u, with max(z, 0) as a median (no NaN-quieting
    // instruction in front of it, as fmaxf would need)
    return fmaf(-fabsf(z), u, __builtin_amdgcn_fmed3f(z, 0.f, 3.0e38f));
}

template <typename T>
__device__ __forceinline__ float gelu_erf(float z) {
    if constexpr (sizeof(T) == 4) return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
    else return gelu_as7126(z);
}

// Registers that carry one K step of the W tile from global memory to LDS.
template <int WF> struct BRegs;
template <> struct BRegs<DT_F32> { uint4 v[4]; };   // dense: same as A
template <> struct BRegs<DT_Q8_0> { uint4 q[2]; float d[2]; };
template <> struct BRegs<DT_Q4_0> { uint4 q; float d; };

template <typename T>
__device__ __forceinline__ void store_f16x8(unsigned char *dst, const float *x) {
    // x holds 8 f32 values, stored as 8 act-dtype values (16 bytes)
    *(uint4 *)dst = make_uint4(pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]), pack2<T>(x[4], x[5]),
                               pack2<T>(x[6], x[7]));
}

// Raw buffer resource over the first nbytes at p (gfx9 descriptor word 3):
// loads past the end return 0 and stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)nbytes, 0x00020000);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The v columns of the qkv product, written transposed: V^T [B, heads, 64,
// npad] holds, for every head and dim, the item's tokens in a row (token n at
// vt_pos(n)).  Each
// 32-row block (32 consecutive tokens, possibly of two items) is finished in
// registers (rounding) and staged in LDS as in the STORE case, then read
// back by column: a wave store writes two columns of 32 tokens, i.e. two runs
// of 64 (2-byte types) or 128 bytes of V^T, one element per lane.  Rows past
// M fall past the end of V^T, where the buffer resource drops them.
template <typename T, int MB_, int NB_>
__device__ __forceinline__ void epilogue_wave_vt(const GemmArgs &g, const f32x16 (&acc)[MB_][NB_],
                                                 unsigned char *ls, int64_t row0,
                                                 int64_t col0, int lane) {
    constexpr int OES = (int)sizeof(T);
    constexpr int RB = 32 * NB_ * OES;
    constexpr int CH = RB / 16;
    constexpr int SWM = (CH < 16 ? CH : 16) - 1;
    const int heads = (int)((g.N - g.vcol0) / 64);
    const int64_t nitems = g.M / g.ntok;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g.vt, (uint32_t)(nitems * heads * 64 * g.npad * OES));
    const int rl = lane & 31, g32 = lane >> 5;
    const int64_t dcol0 = col0 - g.vcol0;        // first v column of the wave (multiple of 64)
#pragma unroll
    for (int i = 0; i < MB_; ++i) {
        // stage block row i (rounding), row-major with swizzled chunks
#pragma unroll
        for (int j = 0; j < NB_; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 32 * j + 8 * q + 4 * g32;
                const float z[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                const int cb = col * OES;
                unsigned char *dst = ls + rl * RB + (((cb >> 4) ^ (rl & SWM)) << 4) + (cb & 15);
                if constexpr (OES == 2) {
                    *(uint2 *)dst = make_uint2(pack2<T>(z[0], z[1]), pack2<T>(z[2], z[3]));
                } else {
                    *(float4 *)dst = make_float4(z[0], z[1], z[2], z[3]);
                }
            }
        // this lane's token: row row0 + 32 i + rl, at its V^T position
        const uint32_t m = (uint32_t)(row0 + 32 * i + rl);
        const uint32_t b = m / (uint32_t)g.ntok, n = m - b * (uint32_t)g.ntok;
        const uint32_t tok = b * (uint32_t)(heads * 64 * g.npad) + (uint32_t)vt_pos(n);   // (b, h=0, d=0, n)
#pragma unroll
        for (int t = 0; t < NB_ * 16; ++t) {
            const int c = 2 * t + g32;                           // column of the wave
            const int cb = c * OES;
            const unsigned char *src = ls + rl * RB + (((cb >> 4) ^ (rl & SWM)) << 4) + (cb & 15);
            const int64_t dc = dcol0 + c;                        // v column: head dc / 64, dim dc % 64
            const uint32_t off = (tok + (uint32_t)dc * (uint32_t)g.npad) * OES;
            if constexpr (OES == 2)
                __builtin_amdgcn_raw_buffer_store_b16(*(const unsigned short *)src, rs, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(*(const unsigned int *)src, rs, off, 0, 0);
        }
    }
}

// The v columns of the qkv product written to V^T straight from the
// accumulators, when the MFMAs took the token operand first: element 4q + r
// of block (i, j) of lane l is token row 32 i + 8 q + 4 (l / 32) + r of the
// wave's tile and v column 32 j + l % 32.  Tokens are aligned in runs of 16
// within their item (items a multiple of 16 tokens long, or one item), and
// a V^T row holds each run as tokens 0-3, 8-11, 4-7, 12-15: so the two
// 4-token groups q = 2h, 2h + 1 of a lane are 8 consecutive positions of
// its column's V^T row, stored as one 16-byte vector.  A run that crosses
// M (the one item's last, when it is not a multiple of 16 long) is stored
// element by element for the tokens below M: V^T's free positions stay
// untouched.  Runs past M fall past the end of V^T and are dropped.
template <typename T, int MB_, int NB_>
__device__ __forceinline__ void epilogue_vt_direct(const GemmArgs &g, const f32x16 (&acc)[MB_][NB_],
                                                   int64_t row0, int64_t col0, int lane) {
    constexpr int OES = (int)sizeof(T);
    static_assert(OES == 2, "16-bit V^T");
    const int64_t D = g.N - g.vcol0;
    const int64_t nitems = g.M / g.ntok;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g.vt, (uint32_t)(nitems * D * g.npad * OES));
    const int cl = lane & 31, g32 = lane >> 5;
#pragma unroll
    for (int j = 0; j < NB_; ++j) {
        const uint32_t dc = (uint32_t)(col0 + 32 * j + cl - g.vcol0);   // V^T row within an item
#pragma unroll
        for (int i = 0; i < MB_; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t ms = (uint32_t)(row0 + 32 * i + 16 * h);    // the run's first token row
                const uint32_t b = ms / (uint32_t)g.ntok, ns = ms - b * (uint32_t)g.ntok;
                const uint32_t off = ((b * (uint32_t)D + dc) * (uint32_t)g.npad + ns + 8 * g32) * OES;
                float x[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[r] = acc[i][j][4 * (2 * h) + r];
                    x[4 + r] = acc[i][j][4 * (2 * h + 1) + r];
                }
                if (ms + 16 <= (uint32_t)g.M || ms >= (uint32_t)g.M) {
                    const u32x4 v = {pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]), pack2<T>(x[4], x[5]),
                                     pack2<T>(x[6], x[7])};
                    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        // position 8 g32 + e of the run holds token (e < 4 ? e : e + 4) + 4 g32
                        const uint32_t tok = ms + 4 * g32 + (e < 4 ? e : e + 4);
                        if (tok < (uint32_t)g.M)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                __builtin_bit_cast(unsigned short, from_f32<T>(x[e])), rs, off + 2 * e, 0, 0);
                    }
                }
            }
    }
}

// The output stage of one wave's MB_ x NB_ accumulator blocks (STORE / GELU
// / RESID / PATCH / QKV), which already include the biases (the K loops
// start from them).  The blocks are accumulated transposed (the weights are the
// MFMA's A operand): element 4q + r of block (i, j) of lane l is output row
// 32 i + l % 32, column 32 j + 8 q + 4 (l / 32) + r of the wave's tile.  Each
// 32-row block is finished in registers (GELU, rounding), written to
// the wave's LDS scratch, and read back so that consecutive lanes hold
// consecutive 16 bytes of a row: every global access then covers whole
// 128-byte lines (32 partial-line writes per row, the register layout's
// pattern, cost more than the rows' bandwidth).  Scratch rows hold 16-byte
// chunk c at c ^ (row % min(16, chunks per row)), which spreads the column
// writes over the banks and keeps the row reads conflict-free.  Outputs go through a buffer resource sized to M rows, so
// rows past M need no branch.  RESID reads X one block ahead of its writes
// (issued after the block's staging, to keep one buffer live there), and each
// element is read and written by one lane only.
template <typename T, int EPI, int MB_, int NB_, bool NO_VT = false>
__device__ __forceinline__ void epilogue_wave(const GemmArgs &g, const f32x16 (&acc)[MB_][NB_],
                                              unsigned char *ls, int64_t row0,
                                              int64_t col0, int lane) {
    if constexpr (EPI == EPI_QKV && !NO_VT) {   // (NO_VT: the caller writes v columns itself)
        // a wave's columns are all q/k or all v (v starts at a multiple of 128)
        if (col0 >= g.vcol0) {
            epilogue_wave_vt<T, MB_, NB_>(g, acc, ls, row0, col0, lane);
            return;
        }
    }
    constexpr int OES = (EPI == EPI_RESID || EPI == EPI_PATCH) ? 4 : (int)sizeof(T);
    constexpr int RB = 32 * NB_ * OES;           // bytes of one scratch row
    constexpr int CH = RB / 16;                  // 16-byte chunks per row = lanes per row
    constexpr int RPI = 64 / CH;                 // rows per read instruction
    constexpr int NRD = 32 / RPI;                // read instructions per 32-row block
    constexpr int SWM = (CH < 16 ? CH : 16) - 1; // chunk swizzle mask
    static_assert(CH <= 64 && 64 % CH == 0, "scratch row shape");
    // EPI_PATCH writes row b*np + n to row b*ntok + has_cls + n of an
    // output of (M / np) * ntok rows, adding pos row has_cls + n
    const uint32_t out_rows = EPI == EPI_PATCH ? (uint32_t)(g.M / g.np * g.ntok) : (uint32_t)g.M;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g.out, (uint32_t)(out_rows * g.ldo * OES));
    const __amdgpu_buffer_rsrc_t rpos = buffer_rsrc(EPI == EPI_PATCH ? g.pos : nullptr,
                                                    EPI == EPI_PATCH && g.pos ? (uint32_t)(g.ntok * g.ldo * 4) : 0u);
    const int rl = lane & 31, g32 = lane >> 5;
    const int rr = lane / CH, rc = lane % CH;     // read side: row in instruction, chunk
    const uint32_t rowb = (uint32_t)(g.ldo * OES);
    // global byte offset of (row0 + 32 i + t*RPI + rr, col0 + 16 rc / OES)
    const uint32_t gbase = (uint32_t)(row0 * g.ldo * OES + col0 * OES) + rr * rowb + rc * 16;

    // EPI_QKV: the q columns' scale, per 4-column group (D is a multiple of 64)
    auto col_scale = [&](int col) -> float {
        if constexpr (EPI == EPI_QKV) {
            if (g.qscale != 0.f && col0 + col < g.vcol0 / 2) return g.qscale;
        }
        return 1.f;
    };
    // RESID: X, PATCH: the pos rows (and the mapped output rows), read one
    // block ahead of their use
    float4 xv[2][NRD];
    uint32_t pout[EPI == EPI_PATCH ? 2 : 1][EPI == EPI_PATCH ? NRD : 1];
    auto load_x = [&](int i, int bf) {
        if constexpr (EPI == EPI_RESID) {
#pragma unroll
            for (int t = 0; t < NRD; ++t)
                xv[bf][t] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                    rs, gbase + (32 * i + t * RPI) * rowb, 0, 0));
        }
        if constexpr (EPI == EPI_PATCH) {
            // rows past M map past the output's end, where the store is dropped
            const uint32_t cb = (uint32_t)(col0 * 4) + rc * 16;
#pragma unroll
            for (int t = 0; t < NRD; ++t) {
                const uint32_t m = (uint32_t)(row0 + 32 * i + t * RPI + rr);
                const uint32_t b = m / (uint32_t)g.np, n = m - b * (uint32_t)g.np;
                const uint32_t t_ = (uint32_t)g.has_cls + n;
                pout[bf][t] = (b * (uint32_t)g.ntok + t_) * rowb + cb;
                xv[bf][t] = g.pos ? __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rpos, t_ * rowb + cb, 0, 0))
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    load_x(0, 0);
#pragma unroll
    for (int i = 0; i < MB_; ++i) {
        __builtin_amdgcn_sched_barrier(0);       // keep the loads where they are issued
        // stage block row i; the rotary branch of EPI_QKV is taken per block
        // row, outside the element loop, so that the loop stays one block
        auto stage = [&](auto ROPE) __attribute__((always_inline)) {
        constexpr bool rope = decltype(ROPE)::value;
        // with rotary position: this lane's token (rows past M wrap to a
        // valid table row; they are dropped at the store)
        uint32_t rn = 0;
        if constexpr (rope) rn = (uint32_t)(row0 + 32 * i + rl) % (uint32_t)g.ntok;
#pragma unroll
        for (int j = 0; j < NB_; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 32 * j + 8 * q + 4 * g32;
                float z[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if constexpr (EPI == EPI_QKV) {
                    if constexpr (rope) {   // dims (d, d+1) and (d+2, d+3) of a head, d % 4 == 0
                        const uint32_t hd = (uint32_t)g.head_dim;
                        const uint32_t p = (uint32_t)((col0 + col) & (hd - 1)) >> 1;
                        const float4 r = *(const float4 *)(g.rope + 2 * (rn * (hd >> 1) + p));
                        const float z0 = z[0], z2 = z[2];
                        z[0] = z0 * r.x - z[1] * r.y;
                        z[1] = z0 * r.y + z[1] * r.x;
                        z[2] = z2 * r.z - z[3] * r.w;
                        z[3] = z2 * r.w + z[3] * r.z;
                    }
                    const float cs = col_scale(col);
#pragma unroll
                    for (int r = 0; r < 4; ++r) z[r] *= cs;
                }
                if constexpr (EPI == EPI_GELU) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) z[r] = gelu_erf<T>(z[r]);
                }
                const int cb = col * OES;
                unsigned char *dst = ls + rl * RB + (((cb >> 4) ^ (rl & SWM)) << 4) + (cb & 15);
                if constexpr (OES == 2) {
                    *(uint2 *)dst = make_uint2(pack2<T>(z[0], z[1]), pack2<T>(z[2], z[3]));
                } else {
                    *(float4 *)dst = make_float4(z[0], z[1], z[2], z[3]);
                }
            }
        };
        if (EPI == EPI_QKV && g.rope)
            stage(std::true_type{});
        else
            stage(std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < MB_) load_x(i + 1, (i + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        // read back by rows and write whole lines
#pragma unroll
        for (int t = 0; t < NRD; ++t) {
            const int r = t * RPI + rr;
            float4 v = *(const float4 *)(ls + r * RB + ((rc ^ (r & SWM)) << 4));
            if constexpr (EPI == EPI_RESID) {
                const float4 x = xv[i & 1][t];
                v.x = x.x + v.x; v.y = x.y + v.y; v.z = x.z + v.z; v.w = x.w + v.w;
            }
            if constexpr (EPI == EPI_PATCH) {
                const float4 q = xv[i & 1][t];      // 0 without a pos table
                v.x = v.x + q.x; v.y = v.y + q.y; v.z = v.z + q.z; v.w = v.w + q.w;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, pout[i & 1][t], 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                                       gbase + (32 * i + t * RPI) * rowb, 0, 0);
            }
        }
    }
}

// TS = 2: 128 x 128 tiles (waves of 64 x 64); TS = 1: 64 x 64 tiles (waves
// of 32 x 32, dense weights only), for GEMMs whose 128-wide tiles would
// leave most CUs idle.
template <typename T, int WF, int EPI, int TS, bool IMPL = false>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs g) {
    typedef Mfma<T> MM;
    constexpr int ES = sizeof(T);
    constexpr int BK = 128 / ES;            // elements per K step
    constexpr int VEC = MM::VEC, KC = MM::KC;
    constexpr bool DENSE = (WF == DT_F32);  // DT_F32 here tags "dense, act dtype"
    constexpr int TB = 64 * TS;             // tile rows and columns
    constexpr int WT = 32 * TS;             // wave tile
    static_assert(TS == 2 || (TS == 1 && DENSE), "64-wide tiles: dense weights only");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2][2][TB * ROWB];
    static_assert(4 * 8192 <= 2 * 2 * TB * ROWB, "epilogue scratch");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = g.m_begin + (int64_t)blockIdx.y * TB, n0 = (int64_t)blockIdx.x * TB;
    // K steps [kt0, kt0 + nk): all of K, or split blockIdx.z of a K split
    // (f32 residual GEMMs; the launcher makes every split non-empty)
    const int nk_all = (int)(g.K / BK);
    const bool split = sizeof(T) == 4 && EPI == EPI_RESID && g.ksplit > 1;
    int kt0 = 0, nk = nk_all;
    if (split) {
        const int per = (nk_all + g.ksplit - 1) / g.ksplit;
        kt0 = (int)blockIdx.z * per;
        nk = min(nk_all - kt0, per);
    }

    const unsigned char *A = (const unsigned char *)g.a;
    const unsigned char *W = (const unsigned char *)g.w;

    uint4 areg[4];
    BRegs<WF> breg;

    // Implicit patch-embed (IMPL): the A tile is gathered from the uint8
    // frames.  K chunk q (8 elements, 8 consecutive bytes of one patch row:
    // (patch * 3) % 8 == 0) sits at byte s_koff[q] past a row's patch origin
    // fbase; its elements' channels run (k0 % 3, k0 % 3 + 1, ...), whose
    // affines s_aff[k0 % 3][e] normalise them.  Rows past M read a clamped
    // valid row: they only feed outputs that are never stored.
    static_assert(!IMPL || (sizeof(T) == 2 && TS == 2 && DENSE), "implicit A: 16-bit, 128-wide tiles");
    constexpr int MAX_KCH = 256;                     // K <= 2048
    __shared__ uint32_t s_koff[IMPL ? MAX_KCH : 1];
    __shared__ float2 s_aff[IMPL ? 24 : 1];
    uint32_t fbase[IMPL ? 2 * TS : 1];
    uint2 preg[IMPL ? 2 * TS : 1];
    int a_r0 = 0;
    bool a_pad = false;
    if constexpr (IMPL) {
        const int p = g.patch, p3 = 3 * p, pp3 = p * p3;
        const uint32_t row_b = (uint32_t)g.fW * 3, frame_b = (uint32_t)g.fH * row_b;
        for (int q = tid; q < (int)(g.K / 8); q += 256) {
            const int k0 = 8 * q, dt = k0 / pp3, rem = k0 - dt * pp3, dy = rem / p3, w = rem - dy * p3;
            s_koff[q] = k0 < g.patch_len ? (uint32_t)dt * frame_b + (uint32_t)dy * row_b + (uint32_t)w : 0xffffffffu;
        }
        if (tid < 24) {
            const int ch = (tid / 8 + tid % 8) % 3;
            s_aff[tid] = make_float2(g.pix_scale[ch], g.pix_shift[ch]);
        }
        const int Hp = g.fH / p, Wp = g.fW / p;
#pragma unroll
        for (int i = 0; i < 2 * TS; ++i) {
            int64_t m = m0 + (tid >> 3) + 32 * i;
            if (m >= g.M) m = g.M - 1;
            const uint32_t b = (uint32_t)(m / g.np), n = (uint32_t)(m - (int64_t)b * g.np);
            const uint32_t tt = n / (uint32_t)(Hp * Wp), rr = n - tt * (uint32_t)(Hp * Wp);
            const uint32_t py = rr / (uint32_t)Wp, px = rr - py * (uint32_t)Wp;
            fbase[i] = (b * (uint32_t)g.fT + tt * (uint32_t)g.tubelet) * frame_b + py * (uint32_t)p * row_b +
                       px * (uint32_t)p3;
        }
        __syncthreads();
    }

    auto load_global = [&](int kt) {
        if constexpr (IMPL) {
            const int q = kt * 8 + (tid & 7);
            const uint32_t ko = s_koff[q];
            a_r0 = (8 * q) % 3;
            a_pad = ko == 0xffffffffu;
#pragma unroll
            for (int i = 0; i < 2 * TS; ++i)
                preg[i] = a_pad ? make_uint2(0, 0) : *(const uint2 *)(g.frames + fbase[i] + ko);
        } else {
#pragma unroll
            for (int i = 0; i < 2 * TS; ++i) {
                const int r = (tid >> 3) + 32 * i;
                const int64_t m = m0 + r;
                areg[i] = make_uint4(0, 0, 0, 0);
                if (m < g.M)
                    areg[i] = *(const uint4 *)(A + (m * g.lda + (int64_t)kt * BK) * ES + (tid & 7) * 16);
            }
        }
        if constexpr (DENSE) {
#pragma unroll
            for (int i = 0; i < 2 * TS; ++i) {
                const int r = (tid >> 3) + 32 * i;
                const int64_t n = n0 + r;
                breg.v[i] = make_uint4(0, 0, 0, 0);
                if (n < g.N)
                    breg.v[i] = *(const uint4 *)(W + (n * g.K + (int64_t)kt * BK) * ES + (tid & 7) * 16);
            }
        } else if constexpr (WF == DT_Q8_0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ci = tid + 256 * i, r = ci >> 2, c4 = ci & 3;
                const int64_t n = n0 + r;
                breg.q[i] = make_uint4(0, 0, 0, 0);
                breg.d[i] = 0.f;
                if (n < g.N) {
                    breg.q[i] = *(const uint4 *)(W + n * g.K + (int64_t)kt * 64 + c4 * 16);
                    breg.d[i] = (float)__builtin_bit_cast(_Float16, g.wscale[n * (g.K / 32) + kt * 2 + (c4 >> 1)]);
                }
            }
        } else {  // q4_0
            const int r = tid >> 1, blk = tid & 1;
            const int64_t n = n0 + r;
            breg.q = make_uint4(0, 0, 0, 0);
            breg.d = 0.f;
            if (n < g.N) {
                breg.q = *(const uint4 *)(W + n * (g.K / 2) + ((int64_t)kt * 2 + blk) * 16);
                breg.d = (float)__builtin_bit_cast(_Float16, g.wscale[n * (g.K / 32) + kt * 2 + blk]);
            }
        }
    };

    auto store_lds = [&](int buf) {
        unsigned char *sa = smem[buf][0];
        unsigned char *sb = smem[buf][1];
        if constexpr (IMPL) {
            float sc[8], sh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 v = s_aff[8 * a_r0 + e];
                sc[e] = a_pad ? 0.f : v.x;
                sh[e] = a_pad ? 0.f : v.y;
            }
#pragma unroll
            for (int i = 0; i < 2 * TS; ++i) {
                const int r = (tid >> 3) + 32 * i;
                float x[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = fmaf((float)((preg[i].x >> (8 * e)) & 255u), sc[e], sh[e]);
                    x[4 + e] = fmaf((float)((preg[i].y >> (8 * e)) & 255u), sc[4 + e], sh[4 + e]);
                }
                store_f16x8<T>(sa + r * ROWB + (tid & 7) * 16, x);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2 * TS; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *(uint4 *)(sa + r * ROWB + (tid & 7) * 16) = areg[i];
            }
        }
        if constexpr (DENSE) {
#pragma unroll
            for (int i = 0; i < 2 * TS; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *(uint4 *)(sb + r * ROWB + (tid & 7) * 16) = breg.v[i];
            }
        } else if constexpr (WF == DT_Q8_0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ci = tid + 256 * i, r = ci >> 2, c4 = ci & 3;
                const int8_t *q = (const int8_t *)&breg.q[i];
                float x[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) x[j] = breg.d[i] * (float)q[j];
                store_f16x8<T>(sb + r * ROWB + c4 * 32, x);
                store_f16x8<T>(sb + r * ROWB + c4 * 32 + 16, x + 8);
            }
        } else {
            const int r = tid >> 1, blk = tid & 1;
            const uint8_t *q = (const uint8_t *)&breg.q;
            float x[32];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                x[j] = breg.d * (float)((int)(q[j] & 15) - 8);
                x[j + 16] = breg.d * (float)((int)(q[j] >> 4) - 8);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) store_f16x8<T>(sb + r * ROWB + blk * 64 + c * 16, x + 8 * c);
        }
    };

    // The accumulators start from the biases, as in the large tile, so
    // that a row's value does not depend on which tile computed it (a
    // split's partial product starts from 0 and leaves them to the second
    // pass).  Element 4q + r of block (i, j) is column 32 j + 8 q + 4 (lane
    // / 32) + r of the wave's tile; a wave's columns are all below N or all
    // past it (N % 64 == 0).
    f32x16 acc[TS][TS];
    {
        const bool with_bias = !split && n0 + wn * WT < g.N;
        const float *bw = g.bias + n0 + wn * WT;
#pragma unroll
        for (int j = 0; j < TS; ++j) {
            float bv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (with_bias) b4 = *(const float4 *)(bw + 32 * j + 8 * q + 4 * (lane >> 5));
                bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
            }
#pragma unroll
            for (int i = 0; i < TS; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = bv[v];
        }
    }

    const int arow = wm * WT + (lane & 31);
    const int brow = wn * WT + (lane & 31);
    const int kofs = (lane >> 5) * VEC * ES;

    load_global(kt0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_global(kt0 + kt + 1);
        const unsigned char *sa = smem[buf][0];
        const unsigned char *sb = smem[buf][1];
#pragma unroll
        for (int c = 0; c < BK / KC; ++c) {
            typename MM::vec av[TS], bv[TS];
#pragma unroll
            for (int i = 0; i < TS; ++i) {
                av[i] = MM::load(sa + (arow + 32 * i) * ROWB + c * KC * ES + kofs);
                bv[i] = MM::load(sb + (brow + 32 * i) * ROWB + c * KC * ES + kofs);
            }
            // weights as the A operand: the accumulators come out transposed
#pragma unroll
            for (int i = 0; i < TS; ++i)
#pragma unroll
                for (int j = 0; j < TS; ++j) acc[i][j] = MM::mma(bv[j], av[i], acc[i][j]);
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: block (i, j) holds rows m0 + wm*WT + i*32 + lane%32 and
    // columns n0 + wn*WT + j*32 + 8*(v/4) + 4*g + v%4 ----
    if (n0 + wn * WT < g.N) {   // a wave's columns are all in or all out (N % 64 == 0)
        // the loop's last barrier has freed the operand tiles: 8 KB of scratch per wave
        if constexpr (sizeof(T) == 4 && EPI == EPI_RESID) {
            if (split) {   // the partial product, plain f32, into split z's [M, N] slice
                GemmArgs gz = g;
                gz.out = g.kpart + (int64_t)blockIdx.z * g.M * g.N;
                gz.ldo = g.N;
                epilogue_wave<T, EPI_STORE, TS, TS>(gz, acc, &smem[0][0][0] + wave * 8192,
                                                                 m0 + wm * WT, n0 + wn * WT, lane);
                return;
            }
        }
        epilogue_wave<T, EPI, TS, TS>(g, acc, &smem[0][0][0] + wave * 8192,
                                                   m0 + wm * WT, n0 + wn * WT, lane);
    }
}

// ---------------------------------------------------------------------------
// int8 path of q8_0 / q4_0 matrices (the GPU analogue of ggml's integer
// "mmq" products that the Benchmarks page times): activations arrive
// quantised per 32-block (int8 codes + f32 scale per block, see
// launch_quant_act), the weights' codes are int8 (q8_0) or nibbles - 8
// (q4_0, widened to int8 on the way into LDS).  Each 32-wide K block is one
// v_mfma_i32_32x32x32_i8 per 32 x 32 output block, started from zero; its
// int32 result is folded into the f32 accumulators as
//   acc += f32(i32) * (d_a[row, block] * d_w[col, block])
// (three VALU operations per output per block: this, not the matrix core,
// sets the rate on this chip).  Two workgroups share a CU, so one wave's
// MFMAs run under the other's rescale.
//
// Tile, staging and epilogues are gemm_kernel's 128 x 128 form (4 waves of
// 64 x 64, 128-byte K steps = 4 blocks, LDS rows padded to 144 bytes, next
// step's loads held in registers); each K step also stages the 128 rows'
// activation scales and weight scales, [block][row] in f32.  The operand
// bytes read per lane follow the same layout for both operands, so the K
// order inside a block is whatever the instruction takes, identically for
// both, and each block's integer dot product is exact.
// ---------------------------------------------------------------------------
typedef signed char i8x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <typename T, int WF, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_i8_kernel(const GemmArgs g) {
    static_assert(sizeof(T) == 2 && (WF == DT_Q8_0 || WF == DT_Q4_0), "16-bit outputs, block weights");
    constexpr int TB = 128, WT = 64;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2][2][TB * ROWB];
    __shared__ __attribute__((aligned(16))) float s_sc[2][2][4][TB];   // [buf][a / w][block][row]
    static_assert(4 * 8192 <= 2 * 2 * TB * ROWB, "epilogue scratch");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = g.m_begin + (int64_t)blockIdx.y * TB, n0 = (int64_t)blockIdx.x * TB;
    const int nk = (int)(g.K / 128);
    const int64_t nb = g.K / 32;
    const unsigned char *A = (const unsigned char *)g.a;
    const unsigned char *W = (const unsigned char *)g.w;

    uint4 areg[4], wreg[4];
    float2 asc;
    uint32_t wsc;
    // scales: thread t carries blocks 2 (t & 1), +1 of row t >> 1
    const int sr = tid >> 1, sb = 2 * (tid & 1);
    auto load_global = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            const int64_t m = m0 + r;
            areg[i] = make_uint4(0, 0, 0, 0);
            if (m < g.M) areg[i] = *(const uint4 *)(A + m * g.lda + (int64_t)kt * 128 + (tid & 7) * 16);
        }
        if constexpr (WF == DT_Q8_0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 3) + 32 * i;
                const int64_t n = n0 + r;
                wreg[i] = make_uint4(0, 0, 0, 0);
                if (n < g.N) wreg[i] = *(const uint4 *)(W + n * g.K + (int64_t)kt * 128 + (tid & 7) * 16);
            }
        } else {   // (row, block) pairs tid and tid + 256: 16 bytes of nibbles each
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int p = tid + 256 * i, r = p >> 2, blk = p & 3;
                const int64_t n = n0 + r;
                wreg[i] = make_uint4(0, 0, 0, 0);
                if (n < g.N) wreg[i] = *(const uint4 *)(W + n * (g.K / 2) + (int64_t)kt * 64 + blk * 16);
            }
        }
        {
            const int64_t m = m0 + sr, n = n0 + sr;
            asc = make_float2(0.f, 0.f);
            wsc = 0;
            if (m < g.M) asc = *(const float2 *)(g.ascale + m * nb + (int64_t)kt * 4 + sb);
            if (n < g.N) wsc = *(const uint32_t *)(g.wscale + n * nb + (int64_t)kt * 4 + sb);
        }
    };
    // q4_0 nibble c -> int8 c - 8, four per word: (c + 0x78) ^ 0x80 per byte
    auto widen4 = [](uint32_t w) -> uint32_t { return ((w & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u; };
    auto store_lds = [&](int buf) {
        unsigned char *sa = smem[buf][0];
        unsigned char *sw = smem[buf][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            *(uint4 *)(sa + r * ROWB + (tid & 7) * 16) = areg[i];
        }
        if constexpr (WF == DT_Q8_0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *(uint4 *)(sw + r * ROWB + (tid & 7) * 16) = wreg[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int p = tid + 256 * i, r = p >> 2, blk = p & 3;
                const uint4 q = wreg[i];
                // byte j of a block: code j (low nibble), code j + 16 (high)
                *(uint4 *)(sw + r * ROWB + blk * 32) = make_uint4(widen4(q.x), widen4(q.y), widen4(q.z), widen4(q.w));
                *(uint4 *)(sw + r * ROWB + blk * 32 + 16) =
                    make_uint4(widen4(q.x >> 4), widen4(q.y >> 4), widen4(q.z >> 4), widen4(q.w >> 4));
            }
        }
        s_sc[buf][0][sb][sr] = asc.x;
        s_sc[buf][0][sb + 1][sr] = asc.y;
        s_sc[buf][1][sb][sr] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wsc & 0xffffu));
        s_sc[buf][1][sb + 1][sr] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wsc >> 16));
    };

    // accumulators start from the biases (gemm_kernel's layout: element
    // 4q + r of block (i, j) is row 32 i + lane % 32, column 32 j + 8 q +
    // 4 (lane / 32) + r of the wave's tile)
    f32x16 acc[2][2];
    {
        const bool with_bias = n0 + wn * WT < g.N;
        const float *bw = g.bias + n0 + wn * WT;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float bv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (with_bias) b4 = *(const float4 *)(bw + 32 * j + 8 * q + 4 * (lane >> 5));
                bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = bv[v];
        }
    }

    const int arow = wm * WT + (lane & 31);
    const int brow = wn * WT + (lane & 31);
    const int kofs = (lane >> 5) * 16;
    const int ccol = wn * WT + 4 * (lane >> 5);   // first scale column of the lane
    const i32x16 zero = {};

    // one block's rescale: acc[i][j] += f32(t[i][j]) * d_a[row] * d_w[col]
    auto rescale = [&](const i32x16 (&t)[2][2], const float (*sc)[4][TB], int c) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float da = sc[0][c][arow + 32 * i];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 dw = *(const float4 *)&sc[1][c][ccol + 32 * j + 8 * q];
                    const float s4[4] = {da * dw.x, da * dw.y, da * dw.z, da * dw.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][j][4 * q + r] = fmaf((float)t[i][j][4 * q + r], s4[r], acc[i][j][4 * q + r]);
                }
        }
    };

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_global(kt + 1);
        const unsigned char *sa = smem[buf][0];
        const unsigned char *sw = smem[buf][1];
        const float (*sc)[4][TB] = s_sc[buf];
        // one block per iteration, not unrolled: unrolled, the compiler
        // hoists every block's scale reads and MFMAs and spills their results
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {
            i8x16 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                av[i] = *(const i8x16 *)(sa + (arow + 32 * i) * ROWB + c * 32 + kofs);
                bv[i] = *(const i8x16 *)(sw + (brow + 32 * i) * ROWB + c * 32 + kofs);
            }
            // weights as the A operand: the accumulators come out transposed
            i32x16 t[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) t[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv[j], av[i], zero, 0, 0, 0);
            rescale(t, sc, c);
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    if (n0 + wn * WT < g.N)   // a wave's columns are all in or all out (N % 64 == 0)
        epilogue_wave<T, EPI, 2, 2>(g, acc, &smem[0][0][0] + wave * 8192, m0 + wm * WT, n0 + wn * WT, lane);
}

template <typename T, int WF>
hipError_t launch_i8_epi(int epi, const GemmArgs &g, hipStream_t s) {
    const dim3 grid((unsigned)cdiv(g.N, 128), (unsigned)cdiv(g.M, 128));
    switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL((gemm_i8_kernel<T, WF, EPI_STORE>), grid, dim3(256), 0, s, g); break;
        case EPI_GELU: hipLaunchKernelGGL((gemm_i8_kernel<T, WF, EPI_GELU>), grid, dim3(256), 0, s, g); break;
        case EPI_RESID: hipLaunchKernelGGL((gemm_i8_kernel<T, WF, EPI_RESID>), grid, dim3(256), 0, s, g); break;
        case EPI_QKV: hipLaunchKernelGGL((gemm_i8_kernel<T, WF, EPI_QKV>), grid, dim3(256), 0, s, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large-tile variant for the encoder's big dense GEMMs: 256 x BN outputs per
// workgroup of 4 waves (2 x 2), each wave 128 x BN/2 (4 x BN/64 blocks of
// 32 x 32 accumulators, held in AGPRs), one workgroup per CU.
//
// K steps of 64 elements (128 bytes of every operand row) flow through a
// ring of NS LDS stages, filled by direct global -> LDS loads
// (global_load_lds_dwordx4: lane i of a wave instruction lands at base +
// 16 i) issued NS - 1 steps ahead.  Eight lanes cover one row's 128 bytes, so
// every L2 request is a whole line: with 64-byte row pieces the L2 request
// rate, not its bandwidth, capped the loads (measured on MI355X: half the
// requests at the same bytes and misses as a vendor GEMM).  A step waits for
// its own stage only, and a stage is refilled only after the barrier that
// follows every wave's last read of it.
//
// LDS rows are 128 bytes with no padding; 16-byte chunk c of row r lives in
// slot c ^ swz(r), swz(r) = (r ^ ((r >> 3) & 3)) & 7, so the rows one operand
// read touches per LDS cycle fall in distinct banks.
//
// Tile order: workgroups go to the 8 XCDs round-robin, so ids are remapped to
// give each XCD a contiguous range of tiles, and within that range GROUP_M
// M-tiles are swept together across N, for L2 reuse of both operands.
// ---------------------------------------------------------------------------
constexpr int BIG_BM = 256;
constexpr int BIG_BK = 64;               // elements per K step (128 bytes of a row)
constexpr int GROUP_M = 4;
constexpr int N_XCD = 8;

// depends on row bits 0-4 only, so a 32-row MFMA block shares one swizzle
__device__ __forceinline__ int swz8(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

__device__ __forceinline__ int xcd_remap(int w, int T) {
    const int q = T / N_XCD, r = T % N_XCD;
    const int x = w % N_XCD, local = w / N_XCD;
    return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// Instruction order inside one K chunk of MBNB MFMAs: NDS LDS reads, two per
// slot, behind the first MFMAs, and NVM global -> LDS loads spread evenly over
// the chunk (one slot = one MFMA and what is issued after it).
template <int ID, int MBNB, int NDS, int NVM, int I>
__device__ __forceinline__ void sched_slot() {
    constexpr int ds = I < NDS / 2 ? 2 : 0;
    constexpr int vm = (I + 1) * NVM / MBNB - I * NVM / MBNB;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);
    if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, ID);
    if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, ID);
}
template <int ID, int MBNB, int NDS, int NVM, int... I>
__device__ __forceinline__ void sched_chunk_seq(std::integer_sequence<int, I...>) {
    (sched_slot<ID, MBNB, NDS, NVM, I>(), ...);
    __builtin_amdgcn_sched_barrier(0);
}
template <int ID, int MBNB, int NDS, int NVM>
__device__ __forceinline__ void sched_chunk() {
    sched_chunk_seq<ID, MBNB, NDS, NVM>(std::make_integer_sequence<int, MBNB>{});
}

template <typename T, int EPI, int BN, bool VTD = false>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(const GemmArgs g, int tiles_m, int tiles_n) {
    typedef Mfma<T> MM;
    typedef typename MM::vec vec;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int NB = BN / 64;                      // 32-column blocks per wave
    constexpr int NS = BN == 256 ? 2 : 3;            // stages: 64 KB or 48 KB each
    constexpr int A_BYTES = BIG_BM * 128, B_BYTES = BN * 128, ST = A_BYTES + B_BYTES;
    constexpr int A_CH = BIG_BM * 8 / 256, B_CH = BN * 8 / 256;   // 16-byte chunks per thread
    constexpr int LPS = A_CH + B_CH;                 // loads per thread per stage
    constexpr int HALF = LPS / 2;
    static_assert(LPS % 2 == 0 && NS * ST <= 160 * 1024, "LDS");
    static_assert((NS - 1) * LPS < 64, "vmcnt range");
    // One array per stage: the compiler gives each its own alias scope, so a
    // read of one stage needs no wait for loads still landing in another (a
    // single indexed array makes it wait for every load in flight).
    __shared__ __attribute__((aligned(1024))) unsigned char lds0[ST];
    __shared__ __attribute__((aligned(1024))) unsigned char lds1[ST];
    // (the third stage only where NS = 3: an array no code names takes no LDS)
    __shared__ __attribute__((aligned(1024))) unsigned char lds2[ST];
    auto stage = [&](auto S) -> unsigned char * __attribute__((always_inline)) {
        if constexpr (decltype(S)::value == 0) return lds0;
        else if constexpr (decltype(S)::value == 1) return lds1;
        else return lds2;
    };
    auto stage_rt = [&](int s) -> unsigned char * __attribute__((always_inline)) {
        if constexpr (NS == 3) return s == 0 ? lds0 : s == 1 ? lds1 : lds2;
        else return s == 0 ? lds0 : lds1;
    };

    const int tid = threadIdx.x, lane = tid & 63, g32 = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS-load bases in SGPRs
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = tiles_m * tiles_n;
    const int pid = xcd_remap((int)blockIdx.x, ntiles);
    const int group = pid / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % (GROUP_M * tiles_n)) % gm;
    const int tn = (pid % (GROUP_M * tiles_n)) / gm;
    const int64_t m0 = g.m_begin + (int64_t)tm * BIG_BM, n0 = (int64_t)tn * BN;
    const int nk = (int)(g.K / BIG_BK);

    const unsigned char *A = (const unsigned char *)g.a;
    const unsigned char *W = (const unsigned char *)g.w;

    // 32-bit byte offsets of this thread's chunks (a K step is a uniform
    // 128-byte advance).  Load l < A_CH is A chunk ci = l*256 + tid, load
    // l >= A_CH is W chunk ci = (l - A_CH)*256 + tid; chunk ci -> row ci >> 3,
    // slot ci & 7, which holds global chunk slot ^ swz(row).  Rows past M / N
    // read a clamped valid row: they only feed outputs that are never stored.
    uint32_t off[LPS];
#pragma unroll
    for (int l = 0; l < LPS; ++l) {
        const bool is_a = l < A_CH;
        const int ci = (is_a ? l : l - A_CH) * 256 + tid, r = ci >> 3, c = (ci & 7) ^ swz8(r);
        if (is_a) {
            int64_t m = m0 + r;
            if (m >= g.M) m = g.M - 1;
            off[l] = (uint32_t)(m * g.lda * 2 + c * 16);
        } else {
            int64_t n = n0 + r;
            if (n >= g.N) n = g.N - 1;
            off[l] = (uint32_t)(n * g.K * 2 + c * 16);
        }
    }
    // half h of the loads of step kt into stage memory st; a stage's loads go
    // out in two halves, so that the CU's address unit is never handed more
    // than it drains while the MFMAs around them run
    auto issue_half = [&](unsigned char *st, int kt, int h) __attribute__((always_inline)) {
#pragma unroll
        for (int l = h * HALF; l < (h + 1) * HALF; ++l) {
            const bool is_a = l < A_CH;
            __builtin_amdgcn_global_load_lds((const void *)((is_a ? A : W) + (size_t)kt * 128 + off[l]),
                (__attribute__((address_space(3))) void *)(st + (is_a ? 0 : A_BYTES) +
                                                           ((is_a ? l : l - A_CH) * 256 + wave * 64) * 16),
                16, 0, 0);
        }
    };

    // HMC: rows per wave, 128 (the full 256-row tile) or 64 (a half tile: the
    // launch's last row tile when at most its first 128 rows exist, e.g. one
    // 3137-token clip's 13th tile; the four waves then share 128 rows instead
    // of idling on padding)
    auto body = [&](auto SWAPC, auto HMC) __attribute__((always_inline)) {
        constexpr bool SWAP = decltype(SWAPC)::value;
        constexpr int HM = decltype(HMC)::value;
        constexpr int MB = HM / 32, MBNB = MB * NB, NRD = MB + NB;
        static_assert(NRD % 2 == 0 && NRD / 2 <= MBNB && HALF <= MBNB, "chunk schedule");
        // (differing first instructions: the compiler then hoists none of the
        // two shapes' identical bias loads above their branch, where they
        // would stay live across it and spill)
        if constexpr (HM == 64) asm volatile("; half row tile");
        else asm volatile("; full row tile");
        // The accumulators start from the biases (N % BN == 0), so that the
        // epilogue has nothing to add.  Element 4q + r of block (i, j) is
        // column 32 j + 8 q + 4 (lane / 32) + r of the wave's tile, or, with
        // the token operand first (SWAP), column 32 j + lane % 32.
        f32x16 acc[MB][NB];
        {
            const float *bw = g.bias + n0 + wn * (BN / 2);
    #pragma unroll
            for (int j = 0; j < NB; ++j) {
                float bv[16];
                if constexpr (SWAP) {
                    const float b1 = bw[32 * j + (lane & 31)];
    #pragma unroll
                    for (int v = 0; v < 16; ++v) bv[v] = b1;
                } else {
    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 b4 = *(const float4 *)(bw + 32 * j + 8 * q + 4 * g32);
                        bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
                    }
                }
    #pragma unroll
                for (int i = 0; i < MB; ++i)
    #pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = bv[v];
            }
        }

        // operand rows of this lane (same swizzle for every row of a 32-row block)
        const int rl = lane & 31, sw = swz8(rl);
        int arow[MB], brow[NB];
    #pragma unroll
        for (int i = 0; i < MB; ++i) arow[i] = (wm * HM + i * 32 + rl) * 128;
    #pragma unroll
        for (int j = 0; j < NB; ++j) brow[j] = A_BYTES + (wn * (BN / 2) + j * 32 + rl) * 128;

        // Operands move LDS -> registers one 16-element K chunk (of 4 per step)
        // ahead of the MFMAs that use them, in two register sets; the first chunk
        // of step kt+1 is read, after the step's barrier, while the MFMAs of the
        // last chunk of step kt run.
        vec a[2][MB], b[2][NB];                       // [register set][block]
        auto read_chunk = [&](const unsigned char *sm, int c, int buf) __attribute__((always_inline)) {
            const int slot = ((2 * c + g32) ^ sw) << 4;
    #pragma unroll
            for (int i = 0; i < MB; ++i) a[buf][i] = MM::load(sm + arow[i] + slot);
    #pragma unroll
            for (int j = 0; j < NB; ++j) b[buf][j] = MM::load(sm + brow[j] + slot);
        };
        auto mma_chunk = [&](int buf) __attribute__((always_inline)) {
    #pragma unroll
            for (int i = 0; i < MB; ++i)
    #pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if constexpr (SWAP)
                        acc[i][j] = MM::mma(a[buf][i], b[buf][j], acc[i][j]);   // tokens first: V^T layout
                    else
                        acc[i][j] = MM::mma(b[buf][j], a[buf][i], acc[i][j]);   // transposed
                }
        };
        // s_waitcnt lgkmcnt(0) with at most n of this thread's loads in flight
        auto wait_loads = [&](int n) __attribute__((always_inline)) {
            switch (n) {
                case 0: __builtin_amdgcn_s_waitcnt(0x070); break;
                case HALF: __builtin_amdgcn_s_waitcnt(0x070 | (HALF & 15) | ((HALF >> 4) << 14)); break;
                case LPS: __builtin_amdgcn_s_waitcnt(0x070 | (LPS & 15) | ((LPS >> 4) << 14)); break;
                default: __builtin_amdgcn_s_waitcnt(0x070 | ((LPS + HALF) & 15) | (((LPS + HALF) >> 4) << 14)); break;
            }
        };

        // Step kt (stage S = kt % NS, a compile-time constant): chunk 0 carries the
        // second half of step kt+NS-1's loads, chunk 3 (after the barrier that
        // frees stage S) the first half of step kt+NS's.  At the barrier the loads
        // allowed in flight are those of the steps after kt+1.
        auto steady_step = [&](auto S, int kt) __attribute__((always_inline)) {
            constexpr int s = decltype(S)::value;
            unsigned char *cur = stage(S);
            unsigned char *nxt = stage(std::integral_constant<int, (s + 1) % NS>{});
            unsigned char *prv = stage(std::integral_constant<int, (s + NS - 1) % NS>{});
            read_chunk(cur, 1, 1);
            issue_half(prv, kt + NS - 1, 1);
            mma_chunk(0);
            sched_chunk<0, MBNB, NRD, HALF>();
            read_chunk(cur, 2, 0);
            mma_chunk(1);
            sched_chunk<1, MBNB, NRD, 0>();
            read_chunk(cur, 3, 1);
            mma_chunk(0);
            sched_chunk<2, MBNB, NRD, 0>();
            wait_loads((NS - 2) * LPS);               // step kt+1 landed
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_chunk(nxt, 0, 0);
            issue_half(cur, kt + NS, 0);
            mma_chunk(1);
            sched_chunk<3, MBNB, NRD, HALF>();
        };

        // prologue: stages 0 .. NS-2 whole, the first half of stage NS-1
    #pragma unroll
        for (int s0 = 0; s0 < NS - 1; ++s0)
            if (s0 < nk) { issue_half(stage_rt(s0), s0, 0); issue_half(stage_rt(s0), s0, 1); }
        if (NS - 1 < nk) issue_half(stage_rt(NS - 1), NS - 1, 0);
        wait_loads(min(NS - 2, nk - 1) * LPS + (NS - 1 < nk ? HALF : 0));   // step 0 landed
        __builtin_amdgcn_s_barrier();
        read_chunk(lds0, 0, 0);

        // Steady steps (a stage to start) in groups of NS, so that every stage is
        // named at compile time; the loop bodies have no branch around their
        // operand reads (a join with a path that skipped them makes the compiler
        // wait for all of them).
        int kt = 0;
        for (; kt + 2 * NS - 1 < nk; kt += NS) {
            steady_step(std::integral_constant<int, 0>{}, kt);
            steady_step(std::integral_constant<int, 1>{}, kt + 1);
            if constexpr (NS == 3) steady_step(std::integral_constant<int, 2>{}, kt + 2);
        }
        // the remaining steps but the last, with run-time stages (a second set of
        // compile-time bodies here would exhaust the registers)
        for (; kt < nk - 1; ++kt) {
            unsigned char *cur = stage_rt(kt % NS);
            read_chunk(cur, 1, 1);
            if (kt + NS - 1 < nk) issue_half(stage_rt((kt + NS - 1) % NS), kt + NS - 1, 1);
            mma_chunk(0);
            read_chunk(cur, 2, 0);
            mma_chunk(1);
            read_chunk(cur, 3, 1);
            mma_chunk(0);
            wait_loads(min(NS - 2, nk - 2 - kt) * LPS);   // step kt+1 landed
            __builtin_amdgcn_s_barrier();
            read_chunk(stage_rt((kt + 1) % NS), 0, 0);
            if (kt + NS < nk) issue_half(cur, kt + NS, 0);
            mma_chunk(1);
        }
        {
            const unsigned char *cur = stage_rt((nk - 1) % NS);
            read_chunk(cur, 1, 1);
            mma_chunk(0);
            read_chunk(cur, 2, 0);
            mma_chunk(1);
            read_chunk(cur, 3, 1);
            mma_chunk(0);
            mma_chunk(1);
        }

        // every wave has read its last operands: stage 0 becomes output scratch
        static_assert(4 * 64 * BN <= ST, "epilogue scratch");
        __builtin_amdgcn_s_barrier();
        if constexpr (SWAP)
            epilogue_vt_direct<T, MB, NB>(g, acc, m0 + wm * HM, n0 + wn * (BN / 2), lane);
        else
            epilogue_wave<T, EPI, MB, NB, VTD>(g, acc, lds0 + wave * (64 * BN), m0 + wm * HM,
                                                     n0 + wn * (BN / 2), lane);
    };
    // VTD (qkv with vt_direct, launched only when v starts at a multiple of
    // BN, so that every tile is all q / k or all v): the v tiles take the
    // token operand first and write V^T rows straight from the accumulators
    auto rows_body = [&](auto SWAPC) __attribute__((always_inline)) {
        if constexpr (BN == 256) {
            if (m0 + 128 >= g.M) {
                body(SWAPC, std::integral_constant<int, 64>{});
                return;
            }
        }
        body(SWAPC, std::integral_constant<int, 128>{});
    };
    if constexpr (EPI == EPI_QKV && VTD) {
        if (n0 >= g.vcol0) rows_body(std::true_type{});
        else rows_body(std::false_type{});
    } else {
        rows_body(std::false_type{});
    }
}

// Variant choice (below); JEPA_GEMM_VARIANT (small | small64 | big256 | big128) pins it.

// CU count of the current device, queried once per device (threads that
// race to fill an entry store the same value)
int cu_count() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (!n) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// out[m, n] += bias[n] + the splits' partial products, added in split order
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(float *out, int64_t ldo, const float *part, int S,
                                                            int64_t M, int N, const float *bias) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N) return;
    const int64_t m = i / N, n = i - m * N;
    float v = bias[n];
    for (int z = 0; z < S; ++z) v += part[z * M * N + i];
    out[m * ldo + n] += v;
}

template <typename T, int EPI, int BN>
hipError_t launch_big(const GemmArgs &g, hipStream_t s, int64_t tm = 0) {
    // tm: the launch's row tiles (0: enough for rows [m_begin, M))
    if (tm <= 0) tm = cdiv(g.M - g.m_begin, BIG_BM);
    const int64_t tn = cdiv(g.N, BN);
    if constexpr (EPI == EPI_QKV) {
        if (g.vt_direct && g.vcol0 % BN == 0) {
            hipLaunchKernelGGL((gemm_big_kernel<T, EPI, BN, true>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, g,
                               (int)tm, (int)tn);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_big_kernel<T, EPI, BN>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, g, (int)tm, (int)tn);
    return hipGetLastError();
}

template <typename T, int WF, int EPI>
hipError_t launch_t(const GemmArgs &g, hipStream_t s) {
    const int64_t rows = g.M - g.m_begin;          // this launch's rows [m_begin, M)
    if constexpr (EPI == EPI_PATCH && sizeof(T) == 2 && WF == DT_F32) {
        if (g.frames) {   // implicit: the A tile gathered from the frames
            GemmArgs gi = g;
            gi.ksplit = 1;
            dim3 grid((unsigned)cdiv(g.N, BN), (unsigned)cdiv(rows, BM));
            hipLaunchKernelGGL((gemm_kernel<T, WF, EPI, 2, true>), grid, dim3(256), 0, s, gi);
            return hipGetLastError();
        }
    }
    if constexpr (sizeof(T) == 2 && WF == DT_F32 && EPI != EPI_PATCH) {
        const char *v = getenv("JEPA_GEMM_VARIANT");
        const std::string var = v ? v : "";
        // the large kernel addresses operands with 32-bit byte offsets
        const bool big_ok = g.N % 128 == 0 && g.K % BIG_BK == 0 && g.M * g.lda * 2 < (1ll << 32) &&
                            g.N * g.K * 2 < (1ll << 32) && cdiv(g.M, BIG_BM) * cdiv(g.N, 128) < (1ll << 31);
        if (big_ok && var == "big256" && g.N % 256 == 0) return launch_big<T, EPI, 256>(g, s);
        if (big_ok && var == "big128") return launch_big<T, EPI, 128>(g, s);
        // Below ~1024 rows the 128 x 128 tile's larger grid fills the chip
        // better.  Above, the 256-row tiles, 256 or 128 columns wide: by the
        // rounds of workgroups each needs (counting the tiles of the launches
        // expected to run beside this one) times its tile time, a 256 x 128
        // tile taking 0.6 of a 256 x 256 one (measured on MI355X at the ViT-L
        // shapes, epilogues aside).  The wide tile wins whenever the tiles
        // fill several rounds; the narrow one when the wide tiles leave CUs
        // idle (ViT-L/16 images, batch 32: fc2 and out-proj have 100 wide tiles).
        // Short K (<= 512, i.e. <= 8 steps: the 384-wide V-JEPA 2 predictor)
        // stays on the 128 x 128 tile: the large tile's prologue and epilogue,
        // which nothing overlaps at one workgroup per CU, outweigh its K loop
        // (measured 3.60 vs 3.75 ms per predictor-width forward).
        if (big_ok && var.empty() && rows >= 1024 && g.K > 512) {
            const int64_t cus = cu_count(), conc = g.conc > 1 ? g.conc : 1;
            if (g.N % 256 == 0) {
                const int64_t tm = cdiv(rows, BIG_BM), tn = g.N / 256;
                const int64_t r256 = cdiv(tm * tn * conc, cus), r128 = cdiv(tm * (g.N / 128) * conc, cus);
                if (10 * r256 <= 6 * r128) {
                    // A launch of its own (no concurrent parts) whose wide
                    // tiles leave a last round at most 40 % full: the full
                    // rounds' rows keep the wide tiles, and the rows left
                    // over (fewer than a round's worth) take the tiles the
                    // rules here pick for them, in a second launch right
                    // behind.  ViT-L/16 LeVJEPA, batch 4 (12548 rows): fc1
                    // 147.5 us in 4 rounds -> 115.6 us for 12288 rows + 12.2 us
                    // for 260 (MI355X).
                    const int64_t full = tm * tn / cus, last = tm * tn - full * cus;
                    const int64_t tm_main = full * cus / tn;
                    if (conc == 1 && full >= 1 && last > 0 && 10 * last <= 4 * cus && tm_main >= 1 &&
                        tm_main < tm) {
                        hipError_t e = launch_big<T, EPI, 256>(g, s, tm_main);
                        if (e != hipSuccess) return e;
                        GemmArgs gt = g;
                        gt.m_begin = g.m_begin + tm_main * BIG_BM;
                        return launch_t<T, WF, EPI>(gt, s);
                    }
                    return launch_big<T, EPI, 256>(g, s);
                }
            }
            return launch_big<T, EPI, 128>(g, s);
        }
    }
    // Dense GEMMs whose 128-wide tiles would fill fewer than half the CUs
    // (small images, one row per item) take 64-wide tiles: four times the
    // workgroups, each a quarter of the serial MFMA chain.
    if constexpr (WF == DT_F32) {
        const char *v = getenv("JEPA_GEMM_VARIANT");
        const bool pin = v && *v;
        const bool fits = cdiv(rows, 64) < 65535;
        if (fits && ((!pin && 2 * cdiv(rows, BM) * cdiv(g.N, BN) < cu_count()) || (pin && !strcmp(v, "small64")))) {
            dim3 grid((unsigned)cdiv(g.N, 64), (unsigned)cdiv(rows, 64));
            if constexpr (sizeof(T) == 4 && EPI == EPI_RESID) {
                // f32 residual GEMMs with a long K and few tiles: split K into
                // S parts of at least 3 steps (BK = 32), S the largest of 8 / 4 / 2
                // that divides the steps, then add the parts in order
                const int64_t nk = g.K / 32;
                int S = 1;
                for (int c : {8, 4, 2})
                    if (S == 1 && nk % c == 0 && nk / c >= 3 && 4 * grid.x * grid.y * c <= (int64_t)cu_count() * 2) S = c;
                if (g.kpart && g.m_begin == 0 && S > 1 && g.M * g.N < (1ll << 31)) {
                    GemmArgs gs = g;
                    gs.ksplit = S;
                    grid.z = S;
                    hipLaunchKernelGGL((gemm_kernel<T, WF, EPI, 1>), grid, dim3(256), 0, s, gs);
                    hipLaunchKernelGGL(ksplit_reduce_kernel, dim3((unsigned)cdiv(g.M * g.N, 256)), dim3(256), 0, s,
                                       (float *)g.out, g.ldo, g.kpart, S, g.M, (int)g.N, g.bias);
                    return hipGetLastError();
                }
            }
            GemmArgs g1 = g;
            g1.ksplit = 1;
            hipLaunchKernelGGL((gemm_kernel<T, WF, EPI, 1>), grid, dim3(256), 0, s, g1);
            return hipGetLastError();
        }
    }
    GemmArgs g2 = g;
    g2.ksplit = 1;
    dim3 grid((unsigned)cdiv(g.N, BN), (unsigned)cdiv(rows, BM));
    hipLaunchKernelGGL((gemm_kernel<T, WF, EPI, 2>), grid, dim3(256), 0, s, g2);
    return hipGetLastError();
}

template <typename T, int WF>
hipError_t launch_epi(int epi, const GemmArgs &g, hipStream_t s) {
    switch (epi) {
        case EPI_STORE: return launch_t<T, WF, EPI_STORE>(g, s);
        case EPI_GELU: return launch_t<T, WF, EPI_GELU>(g, s);
        case EPI_RESID: return launch_t<T, WF, EPI_RESID>(g, s);
        case EPI_QKV: return launch_t<T, WF, EPI_QKV>(g, s);
        case EPI_PATCH:
            if constexpr (WF == DT_F32) return launch_t<T, WF, EPI_PATCH>(g, s);
            return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

// The output-side contract every GEMM launch checks: the QKV layout, and
// the epilogue's 32-bit buffer offsets and 16-byte vectors.
bool epi_ok(int epi, const GemmArgs &g, int es) {
    if (epi == EPI_QKV) {
        // v starts at a multiple of 128 columns, so no wave straddles q/k and v
        if (!g.vt || g.ntok <= 0 || g.M % g.ntok || g.N % 3 || g.vcol0 != 2 * (g.N / 3) || (g.N / 3) % 64 ||
            g.vcol0 % 128 || g.npad < cdiv(g.ntok, 16) * 16 || ((uintptr_t)g.rope & 15) ||
            (g.rope && g.head_dim != 32 && g.head_dim != 64))
            return false;
        if ((g.M / g.ntok + 1) * (g.N / 3) * g.npad * es >= (1ll << 31)) return false;
    }
    // the epilogue addresses the output through a buffer resource with 32-bit
    // byte offsets (rows up to M + 255 are formed, those past M dropped)
    if (epi != EPI_PATCH && (g.M + 256) * g.ldo * (epi == EPI_RESID ? 4 : es) >= (1ll << 31))
        return false;
    if (32 * g.ldo >= (1ll << 31)) return false;   // in-block row offsets are 32-bit
    if (((uintptr_t)g.bias | (uintptr_t)g.out) & 15) return false;   // 16-byte vectors
    if (epi != EPI_PATCH && (g.ldo * (epi == EPI_RESID ? 4 : es)) % 16) return false;
    return true;
}

}  // namespace

hipError_t launch_gemm(int act_dt, int w_dt, int epi, const GemmArgs &g, hipStream_t s) {
    const int es = act_dt == DT_F32 ? 4 : 2;
    const int64_t bk = 128 / es;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % bk || g.N % 64) return hipErrorInvalidValue;
    if (g.lda < g.K || (epi != EPI_PATCH && g.ldo < g.N)) return hipErrorInvalidValue;
    if (g.M / BM >= 65535) return hipErrorInvalidValue;
    if (epi == EPI_PATCH) {
        if (g.np <= 0 || g.M % g.np || g.ntok < g.np + g.has_cls) return hipErrorInvalidValue;
        // rows up to M + 255 map below 2^32 bytes of output; pos rows are 16-byte vectors
        if (((g.M + 256) / g.np + 1) * g.ntok * g.ldo * 4 >= (1ll << 32) || (g.ldo * 4) % 16 ||
            ((uintptr_t)g.pos & 15))
            return hipErrorInvalidValue;
        if (g.frames) {
            const int64_t p = g.patch, row_b = (int64_t)g.fW * 3;
            const int64_t items = g.M / g.np;
            if (act_dt == DT_F32 || w_dt != act_dt || p <= 0 || g.tubelet <= 0 || g.fH % p || g.fW % p ||
                g.fT % g.tubelet || (3 * p) % 8 || row_b % 8 || ((uintptr_t)g.frames & 7) ||
                g.patch_len != g.tubelet * p * p * 3 || g.K < g.patch_len || g.K / 8 > 256 ||
                g.np != (g.fT / g.tubelet) * (g.fH / p) * (g.fW / p) ||
                items * g.fT * g.fH * row_b >= (1ll << 32))
                return hipErrorInvalidValue;
        }
    }
    if (!epi_ok(epi, g, es)) return hipErrorInvalidValue;
    const bool dense = (w_dt == act_dt);
    if (!dense && (act_dt == DT_F32 || (w_dt != DT_Q8_0 && w_dt != DT_Q4_0) || !g.wscale))
        return hipErrorInvalidValue;
    GemmArgs ga = g;
    ga.m_begin = 0;
    ga.vt_direct = epi == EPI_QKV && (g.ntok % 16 == 0 || g.M == g.ntok);
    if (const char *e = getenv("JEPA_VT_DIRECT"))
        if (!strcmp(e, "0")) ga.vt_direct = 0;
    switch (act_dt) {
        case DT_F32: return launch_epi<float, DT_F32>(epi, ga, s);
        case DT_BF16:
            if (dense) return launch_epi<bf16_t, DT_F32>(epi, ga, s);
            if (w_dt == DT_Q8_0) return launch_epi<bf16_t, DT_Q8_0>(epi, ga, s);
            return launch_epi<bf16_t, DT_Q4_0>(epi, ga, s);
        case DT_F16:
            if (dense) return launch_epi<f16_t, DT_F32>(epi, ga, s);
            if (w_dt == DT_Q8_0) return launch_epi<f16_t, DT_Q8_0>(epi, ga, s);
            return launch_epi<f16_t, DT_Q4_0>(epi, ga, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_i8(int act_dt, int w_dt, int epi, const GemmArgs &g, hipStream_t s) {
    if (act_dt != DT_BF16 && act_dt != DT_F16) return hipErrorInvalidValue;
    if (w_dt != DT_Q8_0 && w_dt != DT_Q4_0) return hipErrorInvalidValue;
    if (epi != EPI_STORE && epi != EPI_GELU && epi != EPI_RESID && epi != EPI_QKV) return hipErrorInvalidValue;
    if (!g.a || !g.w || !g.wscale || !g.ascale || !g.bias || !g.out) return hipErrorInvalidValue;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % 128 || g.N % 64 || g.lda < g.K || g.lda % 16 || g.ldo < g.N)
        return hipErrorInvalidValue;
    if (cdiv(g.M, 128) >= 65535) return hipErrorInvalidValue;
    // 16-byte code rows, 8-byte activation-scale pairs, 4-byte weight-scale pairs
    if (((uintptr_t)g.a | (uintptr_t)g.w) & 15 || ((uintptr_t)g.ascale & 7) || ((uintptr_t)g.wscale & 3))
        return hipErrorInvalidValue;
    if (!epi_ok(epi, g, 2)) return hipErrorInvalidValue;
    GemmArgs ga = g;
    ga.m_begin = 0;
    ga.ksplit = 1;
    ga.vt_direct = 0;
    if (act_dt == DT_BF16)
        return w_dt == DT_Q8_0 ? launch_i8_epi<bf16_t, DT_Q8_0>(epi, ga, s) : launch_i8_epi<bf16_t, DT_Q4_0>(epi, ga, s);
    return w_dt == DT_Q8_0 ? launch_i8_epi<f16_t, DT_Q8_0>(epi, ga, s) : launch_i8_epi<f16_t, DT_Q4_0>(epi, ga, s);
}

}  // namespace jepa
