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
#include "common.hpp"
#include "kernels.hpp"

namespace jepa {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 144;                 // LDS bytes per tile row (128 + pad)
constexpr int TILEB = 128 * ROWB;         // LDS bytes per 128-row tile

__device__ __forceinline__ float gelu_erf(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
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
            acc[0][0] = MM::mma(a0, b0, acc[0][0]);
            acc[0][1] = MM::mma(a0, b1, acc[0][1]);
            acc[1][0] = MM::mma(a1, b0, acc[1][0]);
            acc[1][1] = MM::mma(a1, b1, acc[1][1]);
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    const int g32 = lane >> 5;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (col >= g.N) continue;
        const float bias = g.bias[col];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * g32 + (v & 3);
                if (row >= g.M) continue;
                const float z = acc[i][j][v] + bias;
                if constexpr (EPI == EPI_STORE) {
                    ((T *)g.out)[row * g.ldo + col] = from_f32<T>(z);
                } else if constexpr (EPI == EPI_GELU) {
                    ((T *)g.out)[row * g.ldo + col] = from_f32<T>(gelu_erf(z));
                } else if constexpr (EPI == EPI_RESID) {
                    float *x = (float *)g.out + row * g.ldo + col;
                    *x = *x + z;
                } else {  // EPI_PATCH
                    const int64_t b = row / g.np, n = row - b * g.np;
                    const int64_t t = g.has_cls + n;
                    ((float *)g.out)[(b * g.ntok + t) * g.ldo + col] = z + g.pos[t * g.ldo + col];
                }
            }
        }
    }
}

template <typename T, int WF, int EPI>
hipError_t launch_t(const GemmArgs &g, hipStream_t s) {
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
