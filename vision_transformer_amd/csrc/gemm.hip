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
#include <stdlib.h>

#include <string>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace jepa {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 144;                 // LDS bytes per tile row (128 + pad)
constexpr int TILEB = 128 * ROWB;         // LDS bytes per 128-row tile

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26
// (Hastings' rational approximation): |error| <= 1.5e-7 for all x.  One
// reciprocal and one exponential instead of a library erf; used where the
// result is rounded to a 16-bit type anyway.
__device__ __forceinline__ float erf_as7126(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    p *= t;
    const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
    const float y = fmaf(-p, e, 1.0f);
    return copysignf(y, x);
}

// GELU, erf form: 0.5 z (1 + erf(z / sqrt 2)).  The f32 path keeps the
// library erf; 16-bit outputs use the 7.1.26 approximation.
template <typename T>
__device__ __forceinline__ float gelu_erf(float z) {
    if constexpr (sizeof(T) == 4) return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
    else return 0.5f * z * (1.0f + erf_as7126(z * 0.70710678118654752f));
}

// Registers that carry one K step of the W tile from global memory to LDS.
template <int WF> struct BRegs;
template <> struct BRegs<DT_F32> { uint4 v[4]; };   // dense: same as A
template <> struct BRegs<DT_Q8_0> { uint4 q[2]; float d[2]; };
template <> struct BRegs<DT_Q4_0> { uint4 q; float d; };

template <typename T>
__device__ __forceinline__ void store_f16x8(unsigned char *dst, const float *x) {
    // x holds 8 f32 values, stored as 8 act-dtype values (16 bytes)
    uint4 r;
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = from_f32<T>(x[j]).v;
    r.x = h[0] | ((uint32_t)h[1] << 16);
    r.y = h[2] | ((uint32_t)h[3] << 16);
    r.z = h[4] | ((uint32_t)h[5] << 16);
    r.w = h[6] | ((uint32_t)h[7] << 16);
    *(uint4 *)dst = r;
}

// One output element: z = acc + bias, applied per the epilogue.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &g, int64_t row, int64_t col, float z) {
    if constexpr (EPI == EPI_STORE) {
        ((T *)g.out)[row * g.ldo + col] = from_f32<T>(z);
    } else if constexpr (EPI == EPI_GELU) {
        ((T *)g.out)[row * g.ldo + col] = from_f32<T>(gelu_erf<T>(z));
    } else if constexpr (EPI == EPI_RESID) {
        float *x = (float *)g.out + row * g.ldo + col;
        *x = *x + z;
    } else {  // EPI_PATCH
        const int64_t b = row / g.np, n = row - b * g.np;
        const int64_t t = g.has_cls + n;
        ((float *)g.out)[(b * g.ntok + t) * g.ldo + col] = z + g.pos[t * g.ldo + col];
    }
}

// One 32 x 32 accumulator block of a lane, accumulated transposed (the
// weights are the MFMA's A operand, the activations its B operand): the lane
// owns output row `row` and, for v = 4q + r, column col0 + 8q + r.  Each
// group of 4 consecutive columns is one 8-byte (16-bit out) or 16-byte (f32)
// access, with the 4 biases from one 16-byte load.  STORE / GELU / RESID.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue_block_t(const GemmArgs &g, const f32x16 &acc, int64_t row,
                                                 int64_t col0) {
    if (row >= g.M) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t col = col0 + 8 * q;
        if (col >= g.N) continue;
        const float4 b4 = *(const float4 *)(g.bias + col);
        float z[4] = {acc[4 * q] + b4.x, acc[4 * q + 1] + b4.y, acc[4 * q + 2] + b4.z, acc[4 * q + 3] + b4.w};
        if constexpr (EPI == EPI_RESID) {
            float4 *x = (float4 *)((float *)g.out + row * g.ldo + col);
            float4 v = *x;
            v.x += z[0]; v.y += z[1]; v.z += z[2]; v.w += z[3];
            *x = v;
        } else {
            if constexpr (EPI == EPI_GELU) {
#pragma unroll
                for (int r = 0; r < 4; ++r) z[r] = gelu_erf<T>(z[r]);
            }
            if constexpr (sizeof(T) == 2) {
                uint2 pk;
                pk.x = (uint32_t)from_f32<T>(z[0]).v | ((uint32_t)from_f32<T>(z[1]).v << 16);
                pk.y = (uint32_t)from_f32<T>(z[2]).v | ((uint32_t)from_f32<T>(z[3]).v << 16);
                *(uint2 *)((T *)g.out + row * g.ldo + col) = pk;
            } else {
                *(float4 *)((float *)g.out + row * g.ldo + col) = make_float4(z[0], z[1], z[2], z[3]);
            }
        }
    }
}

template <typename T, int WF, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs g) {
    typedef Mfma<T> MM;
    constexpr int ES = sizeof(T);
    constexpr int BK = 128 / ES;            // elements per K step
    constexpr int VEC = MM::VEC, KC = MM::KC;
    constexpr bool DENSE = (WF == DT_F32);  // DT_F32 here tags "dense, act dtype"

    __shared__ __attribute__((aligned(16))) unsigned char smem[2][2][TILEB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int nk = (int)(g.K / BK);

    const unsigned char *A = (const unsigned char *)g.a;
    const unsigned char *W = (const unsigned char *)g.w;

    uint4 areg[4];
    BRegs<WF> breg;

    auto load_global = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            const int64_t m = m0 + r;
            areg[i] = make_uint4(0, 0, 0, 0);
            if (m < g.M)
                areg[i] = *(const uint4 *)(A + (m * g.lda + (int64_t)kt * BK) * ES + (tid & 7) * 16);
        }
        if constexpr (DENSE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            *(uint4 *)(sa + r * ROWB + (tid & 7) * 16) = areg[i];
        }
        if constexpr (DENSE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
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

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int arow = wm * 64 + (lane & 31);
    const int brow = wn * 64 + (lane & 31);
    const int kofs = (lane >> 5) * VEC * ES;

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_global(kt + 1);
        const unsigned char *sa = smem[buf][0];
        const unsigned char *sb = smem[buf][1];
#pragma unroll
        for (int c = 0; c < BK / KC; ++c) {
            typename MM::vec a0 = MM::load(sa + arow * ROWB + c * KC * ES + kofs);
            typename MM::vec a1 = MM::load(sa + (arow + 32) * ROWB + c * KC * ES + kofs);
            typename MM::vec b0 = MM::load(sb + brow * ROWB + c * KC * ES + kofs);
            typename MM::vec b1 = MM::load(sb + (brow + 32) * ROWB + c * KC * ES + kofs);
            // weights as the A operand: the accumulators come out transposed
            acc[0][0] = MM::mma(b0, a0, acc[0][0]);
            acc[0][1] = MM::mma(b1, a0, acc[0][1]);
            acc[1][0] = MM::mma(b0, a1, acc[1][0]);
            acc[1][1] = MM::mma(b1, a1, acc[1][1]);
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: block (i, j) holds rows m0 + wm*64 + i*32 + lane%32 and
    // columns n0 + wn*64 + j*32 + 8*(v/4) + 4*g + v%4 ----
    const int g32 = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t row = m0 + wm * 64 + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col0 = n0 + wn * 64 + j * 32 + 4 * g32;
            if constexpr (EPI == EPI_PATCH) {
                if (row >= g.M) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t col = col0 + 8 * (v >> 2) + (v & 3);
                    if (col < g.N) epilogue<T, EPI>(g, row, col, acc[i][j][v] + g.bias[col]);
                }
            } else {
                epilogue_block_t<T, EPI>(g, acc[i][j], row, col0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large-tile variant for the encoder's big dense GEMMs: 256 x BN outputs per
// workgroup of 4 waves (2 x 2), each wave 128 x BN/2 (4 x BN/64 blocks of
// 32 x 32 accumulators, held in AGPRs), one workgroup per CU.
//
// K steps of 32 elements flow through a 4-stage LDS ring, filled by direct
// global -> LDS loads (global_load_lds_dwordx4: lane i of a wave instruction
// lands at base + 16 i) issued three steps ahead, so memory latency hides
// behind three steps of MFMAs.  Each step waits for its own stage only
// (vmcnt), reads all of its MFMA operands into registers, and only then issues
// the next stage's loads: no LDS read ever follows a load in flight.
//
// LDS rows are 64 bytes with no padding; chunk c (16 bytes) of row r lives in
// slot c ^ swz(r), swz(r) = ((r >> 1) ^ (r >> 3)) & 3, so the rows one
// operand read touches per LDS cycle fall in distinct banks.
//
// Tile order: workgroups go to the 8 XCDs round-robin, so ids are remapped to
// give each XCD a contiguous range of tiles, and within that range GROUP_M
// M-tiles are swept together across N, for L2 reuse of both operands.
// ---------------------------------------------------------------------------
constexpr int BIG_BM = 256;
constexpr int BIG_BK = 32;               // elements per K step (64 bytes of a row)
constexpr int BIG_NS = 4;                // LDS stages
constexpr int GROUP_M = 4;
constexpr int N_XCD = 8;

__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ int xcd_remap(int w, int T) {
    const int q = T / N_XCD, r = T % N_XCD;
    const int x = w % N_XCD, local = w / N_XCD;
    return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

template <typename T, int EPI, int BN>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(const GemmArgs g, int tiles_m, int tiles_n) {
    typedef Mfma<T> MM;
    typedef typename MM::vec vec;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int MB = 4, NB = BN / 64;              // 32x32 blocks per wave
    constexpr int A_BYTES = BIG_BM * 64, B_BYTES = BN * 64, ST = A_BYTES + B_BYTES;
    constexpr int A_CH = BIG_BM * 4 / 256, B_CH = BN * 4 / 256;   // 16-byte chunks per thread
    __shared__ __attribute__((aligned(1024))) unsigned char smem[BIG_NS * ST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g32 = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = tiles_m * tiles_n;
    const int pid = xcd_remap((int)blockIdx.x, ntiles);
    const int group = pid / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % (GROUP_M * tiles_n)) % gm;
    const int tn = (pid % (GROUP_M * tiles_n)) / gm;
    const int64_t m0 = (int64_t)tm * BIG_BM, n0 = (int64_t)tn * BN;
    const int nk = (int)(g.K / BIG_BK);

    const unsigned char *A = (const unsigned char *)g.a;
    const unsigned char *W = (const unsigned char *)g.w;

    // 32-bit byte offsets of this thread's chunks (a K step is a uniform
    // 64-byte advance).  Chunk id ci = i*256 + tid -> row ci >> 2, slot ci & 3,
    // which holds global chunk slot ^ swz(row).  Rows past M / N read a
    // clamped valid row: they only feed outputs that are never stored.
    uint32_t aoff[A_CH], woff[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int ci = i * 256 + tid, r = ci >> 2, c = (ci & 3) ^ swz4(r);
        int64_t m = m0 + r;
        if (m >= g.M) m = g.M - 1;
        aoff[i] = (uint32_t)(m * g.lda * 2 + c * 16);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int ci = i * 256 + tid, r = ci >> 2, c = (ci & 3) ^ swz4(r);
        int64_t n = n0 + r;
        if (n >= g.N) n = g.N - 1;
        woff[i] = (uint32_t)(n * g.K * 2 + c * 16);
    }
    auto issue = [&](int kt) {
        unsigned char *st = smem + (kt % BIG_NS) * ST;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(A + (size_t)kt * 64 + aoff[i]),
                (__attribute__((address_space(3))) void *)(st + (i * 256 + wave * 64) * 16), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(W + (size_t)kt * 64 + woff[i]),
                (__attribute__((address_space(3))) void *)(st + A_BYTES + (i * 256 + wave * 64) * 16), 16, 0, 0);
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // operand rows of this lane (same swizzle for every row of a 32-row block)
    const int rl = lane & 31, sw = swz4(rl);
    int arow[MB], brow[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) arow[i] = (wm * 128 + i * 32 + rl) * 64;
#pragma unroll
    for (int j = 0; j < NB; ++j) brow[j] = A_BYTES + (wn * (BN / 2) + j * 32 + rl) * 64;

    // Operands move LDS -> registers one K half (16 elements) at a time, two
    // halves in flight: step kt reads its second half while the MFMAs of its
    // first half run, then (after one barrier) the first half of step kt+1
    // while the MFMAs of its second half run.  Before that barrier every wave
    // has finished reading stage kt and step kt+1 has landed, so the barrier
    // both publishes stage kt+1 and frees stage kt for the loads of step
    // kt+NS.
    vec a[2][MB], b[2][NB];                       // [half buffer][block]
    auto read_half = [&](int kt, int c, int buf) {
        const unsigned char *sm = smem + (kt % BIG_NS) * ST;
        const int slot = ((2 * c + g32) ^ sw) << 4;
#pragma unroll
        for (int i = 0; i < MB; ++i) a[buf][i] = MM::load(sm + arow[i] + slot);
#pragma unroll
        for (int j = 0; j < NB; ++j) b[buf][j] = MM::load(sm + brow[j] + slot);
    };
    auto mma_half = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[i][j] = MM::mma(b[buf][j], a[buf][i], acc[i][j]);   // transposed
    };
    // s_waitcnt lgkmcnt(0) with at most n stages of loads still in flight
    constexpr int LPS = A_CH + B_CH;              // loads per thread per stage
    auto wait_stages = [&](int n) {
        switch (n) {
            case 0: __builtin_amdgcn_s_waitcnt(0x070); break;
            case 1: __builtin_amdgcn_s_waitcnt(0x070 | (LPS & 15) | ((LPS >> 4) << 14)); break;
            case 2: __builtin_amdgcn_s_waitcnt(0x070 | ((2 * LPS) & 15) | (((2 * LPS) >> 4) << 14)); break;
            default: __builtin_amdgcn_s_waitcnt(0x070 | ((3 * LPS) & 15) | (((3 * LPS) >> 4) << 14)); break;
        }
    };
    static_assert(BIG_NS <= 4 && 3 * (A_CH + B_CH) < 64, "wait_stages encodings");

#pragma unroll
    for (int s0 = 0; s0 < BIG_NS; ++s0)
        if (s0 < nk) issue(s0);
    wait_stages(min(BIG_NS - 1, nk - 1));         // step 0 landed
    __builtin_amdgcn_s_barrier();
    read_half(0, 0, 0);

    for (int kt = 0; kt < nk; ++kt) {
        read_half(kt, 1, 1);
        mma_half(0);
        if (kt + 1 < nk) {
            // issued so far: steps <= min(kt+NS-1, nk-1); step kt+1 must land
            wait_stages(min(BIG_NS - 2, nk - 2 - kt));
            __builtin_amdgcn_s_barrier();
            if (kt + BIG_NS < nk) issue(kt + BIG_NS);
            read_half(kt + 1, 0, 0);
        }
        mma_half(1);
    }

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            epilogue_block_t<T, EPI>(g, acc[i][j], m0 + wm * 128 + i * 32 + rl,
                                     n0 + wn * (BN / 2) + j * 32 + 4 * g32);
}

// Variant choice (below); JEPA_GEMM_VARIANT (small | big256 | big128) pins it.

template <typename T, int EPI, int BN>
hipError_t launch_big(const GemmArgs &g, hipStream_t s) {
    const int tm = (int)cdiv(g.M, BIG_BM), tn = (int)cdiv(g.N, BN);
    hipLaunchKernelGGL((gemm_big_kernel<T, EPI, BN>), dim3(tm * tn), dim3(256), 0, s, g, tm, tn);
    return hipGetLastError();
}

template <typename T, int WF, int EPI>
hipError_t launch_t(const GemmArgs &g, hipStream_t s) {
    if constexpr (sizeof(T) == 2 && WF == DT_F32 && EPI != EPI_PATCH) {
        const char *v = getenv("JEPA_GEMM_VARIANT");
        const std::string var = v ? v : "";
        // the large kernel addresses operands with 32-bit byte offsets
        const bool big_ok = g.N % 128 == 0 && g.K % BIG_BK == 0 && g.M * g.lda * 2 < (1ll << 32) &&
                            g.N * g.K * 2 < (1ll << 32) && cdiv(g.M, BIG_BM) * cdiv(g.N, 128) < (1ll << 31);
        if (big_ok && var == "big256" && g.N % 256 == 0) return launch_big<T, EPI, 256>(g, s);
        if (big_ok && var == "big128") return launch_big<T, EPI, 128>(g, s);
        // measured on MI355X at the ViT-L shapes (M = 12548): the large tile
        // wins when K is long (fc2) or N small (out-proj); for K = 1024 with
        // wide N (qkv, fc1) two 128 x 128 workgroups per CU hide each other's
        // tile prologue and epilogue better
        if (big_ok && var.empty() && g.M >= 1024 && (g.K >= 2048 || g.N <= 1024)) {
            if (g.N % 256 == 0) return launch_big<T, EPI, 256>(g, s);
            return launch_big<T, EPI, 128>(g, s);
        }
    }
    dim3 grid((unsigned)cdiv(g.N, BN), (unsigned)cdiv(g.M, BM));
    hipLaunchKernelGGL((gemm_kernel<T, WF, EPI>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

template <typename T, int WF>
hipError_t launch_epi(int epi, const GemmArgs &g, hipStream_t s) {
    switch (epi) {
        case EPI_STORE: return launch_t<T, WF, EPI_STORE>(g, s);
        case EPI_GELU: return launch_t<T, WF, EPI_GELU>(g, s);
        case EPI_RESID: return launch_t<T, WF, EPI_RESID>(g, s);
        case EPI_PATCH:
            if constexpr (WF == DT_F32) return launch_t<T, WF, EPI_PATCH>(g, s);
            return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int act_dt, int w_dt, int epi, const GemmArgs &g, hipStream_t s) {
    const int es = act_dt == DT_F32 ? 4 : 2;
    const int64_t bk = 128 / es;
    if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % bk || g.N % 64) return hipErrorInvalidValue;
    if (g.lda < g.K || (epi != EPI_PATCH && g.ldo < g.N)) return hipErrorInvalidValue;
    if (g.M / BM >= 65535) return hipErrorInvalidValue;
    if (epi == EPI_PATCH && (g.np <= 0 || g.M % g.np || !g.pos)) return hipErrorInvalidValue;
    if (32 * g.ldo >= (1ll << 31)) return hipErrorInvalidValue;   // in-block row offsets are 32-bit
    const bool dense = (w_dt == act_dt);
    if (!dense && (act_dt == DT_F32 || (w_dt != DT_Q8_0 && w_dt != DT_Q4_0) || !g.wscale))
        return hipErrorInvalidValue;
    switch (act_dt) {
        case DT_F32: return launch_epi<float, DT_F32>(epi, g, s);
        case DT_BF16:
            if (dense) return launch_epi<bf16_t, DT_F32>(epi, g, s);
            if (w_dt == DT_Q8_0) return launch_epi<bf16_t, DT_Q8_0>(epi, g, s);
            return launch_epi<bf16_t, DT_Q4_0>(epi, g, s);
        case DT_F16:
            if (dense) return launch_epi<f16_t, DT_F32>(epi, g, s);
            if (w_dt == DT_Q8_0) return launch_epi<f16_t, DT_Q8_0>(epi, g, s);
            return launch_epi<f16_t, DT_Q4_0>(epi, g, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace jepa
