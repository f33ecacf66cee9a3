// The bandwidth-bound kernels of the encoder: patchify (pixel ingest and
// normalisation), LayerNorm, CLS rows, pooling and dequantisation.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace jepa {
namespace {

// ---------------------------------------------------------------------------
// patchify: uint8 frames [B, T, H, W, 3] -> act [B*Np, ld].  Pixel u of
// channel c becomes (u/255 - mean_c)/std_c; a patch vector lists
// (dt, dy, dx, c) with c fastest; tokens are slot-major then raster.
// Columns P..ld-1 are zero (K padding for the patch-embed GEMM).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const PatchifyArgs a, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int p = a.patch, kt = a.tubelet;
    const int P = kt * p * p * 3;
    const int64_t row = idx / a.ld;
    const int k = (int)(idx - row * a.ld);
    float val = 0.f;
    if (k < P) {
        const int Hp = a.H / p, Wp = a.W / p, Tt = a.T / kt;
        const int64_t np = (int64_t)Tt * Hp * Wp;
        const int64_t b = row / np;
        const int n = (int)(row - b * np);
        const int tt = n / (Hp * Wp), r = n - tt * (Hp * Wp);
        const int i = r / Wp, j = r - i * Wp;
        const int c = k % 3;
        int t2 = k / 3;
        const int dx = t2 % p;
        t2 /= p;
        const int dy = t2 % p, dt = t2 / p;
        const int64_t pix = ((b * a.T + tt * kt + dt) * a.H + i * p + dy) * (int64_t)a.W + j * p + dx;
        const float u = (float)a.frames[pix * 3 + c];
        val = (u / 255.f - a.mean[c]) / a.std[c];
    }
    ((T *)a.out)[idx] = from_f32<T>(val);
}

// The sum over a wave's 64 lanes, returned uniform: within each quad by two
// DPP lane swaps (xor 1, xor 2), within each row of 16 by DPP rotations by 4
// and 8 (every lane then holds its row's sum), then the four rows' sums read
// from lanes 0, 16, 32 and 48 and added in that order.  No LDS round trip,
// unlike the xor shuffles.  Every lane of the wave must be active (the
// LayerNorm kernels give a whole wave to each row).
__device__ __forceinline__ float wave_sum_dpp(float v) {
    auto dpp = [](float x, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                    0xF, 0xF, true));
    };
    v += dpp(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
    v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
    v += dpp(v, std::integral_constant<int, 0x124>{});   // row_ror:4
    v += dpp(v, std::integral_constant<int, 0x128>{});   // row_ror:8
    const int b = __builtin_bit_cast(int, v);
    return ((__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32))) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
}

// ---------------------------------------------------------------------------
// LayerNorm over D = 64*EPL features, one wavefront per row: biased
// variance, eps inside the square root, f32 statistics.
// ---------------------------------------------------------------------------
template <int EPL, typename TO>
__global__ __launch_bounds__(256) void layernorm_kernel(const float *__restrict__ x, int64_t rows,
                                                        const float *__restrict__ gam,
                                                        const float *__restrict__ bet, float eps,
                                                        TO *__restrict__ y) {
    constexpr int D = 64 * EPL;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *xr = x + row * D;
    float v[EPL];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        v[i] = xr[lane + 64 * i];
        s += v[i];
    }
    const float mean = wave_sum_dpp(s) * (1.f / D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float c = v[i] - mean;
        q = fmaf(c, c, q);
    }
    const float rs = rsqrtf(wave_sum_dpp(q) * (1.f / D) + eps);
    TO *yr = y + row * D;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int d = lane + 64 * i;
        yr[d] = from_f32<TO>((v[i] - mean) * rs * gam[d] + bet[d]);
    }
}

// The same LayerNorm for D a multiple of 256, one wavefront per row with
// 16-byte accesses: lane l holds elements 4 l + 256 i + {0..3}.
template <int EV, typename TO>
__global__ __launch_bounds__(256) void layernorm_vec_kernel(const float *__restrict__ x, int64_t rows,
                                                            const float *__restrict__ gam,
                                                            const float *__restrict__ bet, float eps,
                                                            TO *__restrict__ y) {
    constexpr int D = 256 * EV;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float4 *xr = (const float4 *)(x + row * D);
    float4 v[EV];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EV; ++i) v[i] = xr[lane + 64 * i];
#pragma unroll
    for (int i = 0; i < EV; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum_dpp(s) * (1.f / D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < EV; ++i) {
        const float c0 = v[i].x - mean, c1 = v[i].y - mean, c2 = v[i].z - mean, c3 = v[i].w - mean;
        q = fmaf(c0, c0, q);
        q = fmaf(c1, c1, q);
        q = fmaf(c2, c2, q);
        q = fmaf(c3, c3, q);
    }
    const float rs = rsqrtf(wave_sum_dpp(q) * (1.f / D) + eps);
#pragma unroll
    for (int i = 0; i < EV; ++i) {
        const int d = 4 * (lane + 64 * i);
        const float4 gv = *(const float4 *)(gam + d), bv = *(const float4 *)(bet + d);
        const float o0 = (v[i].x - mean) * rs * gv.x + bv.x, o1 = (v[i].y - mean) * rs * gv.y + bv.y;
        const float o2 = (v[i].z - mean) * rs * gv.z + bv.z, o3 = (v[i].w - mean) * rs * gv.w + bv.w;
        if constexpr (sizeof(TO) == 4) {
            *(float4 *)((float *)y + row * D + d) = make_float4(o0, o1, o2, o3);
        } else {
            *(uint2 *)((TO *)y + row * D + d) = make_uint2(pack2<TO>(o0, o1), pack2<TO>(o2, o3));
        }
    }
}

template <typename TO>
hipError_t ln_dispatch(const float *x, int64_t rows, int dim, const float *g, const float *b,
                       float eps, void *y, hipStream_t s) {
    dim3 grid((unsigned)cdiv(rows, 4));
    const char *e = getenv("JEPA_LN_VEC");
    const bool vec = !(e && !strcmp(e, "0")) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)g % 16 == 0) &&
                     ((uintptr_t)b % 16 == 0) && ((uintptr_t)y % 16 == 0);
    if (vec) {
        switch (dim) {
            case 1024: hipLaunchKernelGGL((layernorm_vec_kernel<4, TO>), grid, dim3(256), 0, s, x, rows, g, b, eps, (TO *)y); return hipGetLastError();
            case 768: hipLaunchKernelGGL((layernorm_vec_kernel<3, TO>), grid, dim3(256), 0, s, x, rows, g, b, eps, (TO *)y); return hipGetLastError();
            case 512: hipLaunchKernelGGL((layernorm_vec_kernel<2, TO>), grid, dim3(256), 0, s, x, rows, g, b, eps, (TO *)y); return hipGetLastError();
            case 1280: hipLaunchKernelGGL((layernorm_vec_kernel<5, TO>), grid, dim3(256), 0, s, x, rows, g, b, eps, (TO *)y); return hipGetLastError();
        }
    }
#define LN_CASE(E)                                                                         \
    case E:                                                                                \
        hipLaunchKernelGGL((layernorm_kernel<E, TO>), grid, dim3(256), 0, s, x, rows, g, b, \
                           eps, (TO *)y);                                                  \
        return hipGetLastError();
    switch (dim / 64) {
        LN_CASE(2) LN_CASE(3) LN_CASE(4) LN_CASE(6) LN_CASE(8) LN_CASE(12) LN_CASE(16)
        LN_CASE(20) LN_CASE(24) LN_CASE(32)
    }
#undef LN_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// CLS rows and pooling
// ---------------------------------------------------------------------------
__global__ void cls_rows_kernel(float *x, const float *cls, const float *pos, int N, int D) {
    const int b = blockIdx.x;
    for (int d = threadIdx.x; d < D; d += blockDim.x) x[(int64_t)b * N * D + d] = pos ? cls[d] + pos[d] : cls[d];
}

__global__ void pool_cls_kernel(const float *y, int N, int D, float *out) {
    const int b = blockIdx.x;
    for (int d = threadIdx.x; d < D; d += blockDim.x) out[(int64_t)b * D + d] = y[(int64_t)b * N * D + d];
}

// Mean over rows first..N-1 of item b in two deterministic passes, so that
// a long token map spreads over the whole chip: pass 1 sums chunk ch of the
// rows (POOL_CHUNKS chunks per item) for 64 columns per block, 4 row phases
// per column; pass 2 adds an item's chunk sums in chunk order and divides.
__global__ __launch_bounds__(256) void pool_mean_part_kernel(const float *y, int N, int D, int first,
                                                             float *part) {
    __shared__ float red[256];
    const int b = blockIdx.x, ch = blockIdx.z, tid = threadIdx.x;
    const int d = blockIdx.y * 64 + (tid & 63), phase = tid >> 6;
    const int len = (N - first + POOL_CHUNKS - 1) / POOL_CHUNKS;
    const int r0 = first + ch * len, r1 = min(N, r0 + len);
    const float *yb = y + (int64_t)b * N * D;
    float s = 0.f;
    for (int r = r0 + phase; r < r1; r += 4) s += yb[(int64_t)r * D + d];
    red[tid] = s;
    __syncthreads();
    if (tid < 64)
        part[((int64_t)b * POOL_CHUNKS + ch) * D + d] = (red[tid] + red[tid + 64]) + (red[tid + 128] + red[tid + 192]);
}

__global__ __launch_bounds__(256) void pool_mean_fin_kernel(const float *part, int B, int N, int D, int first,
                                                            float *out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)B * D) return;
    const int64_t b = i / D, d = i - b * D;
    float s = 0.f;
    for (int ch = 0; ch < POOL_CHUNKS; ++ch) s += part[(b * POOL_CHUNKS + ch) * D + d];
    out[i] = s / (float)(N - first);
}

// ---------------------------------------------------------------------------
// Block formats (device layouts in kernels.hpp).  unit_values writes the f32
// values of unit k, 32 consecutive weights of a row; each is the exact value
// rounded once to f32: q8_0 f32(d) q and q4_0 f32(d) (q - 8) (exact);
// q6_K d sc (q - 32) (at most 24 significant bits, exact); q4_K
// d sc_j q - dmin m_j (both products exact, the difference rounded once).
// Formats: jepa.cpp Quantization page, "The rule" and "File sizes" (block
// 32 for q8_0 / q4_0, super-block 256 for the K-quants), with ggml's
// published super-block layouts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_at(const uint16_t *p, int64_t i) {
    return (float)__builtin_bit_cast(_Float16, p[i]);
}

__device__ __forceinline__ void unit_values(int w_dt, const void *codes, const uint16_t *scale,
                                            const uint8_t *sub, int64_t k, float *x) {
    if (w_dt == DT_Q8_0) {
        const float d = half_at(scale, k);
        const uint4 *src = (const uint4 *)((const int8_t *)codes + k * 32);
        const uint4 q0 = src[0], q1 = src[1];
        const int8_t *c0 = (const int8_t *)&q0, *c1 = (const int8_t *)&q1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = d * (float)c0[i];
            x[16 + i] = d * (float)c1[i];
        }
    } else if (w_dt == DT_Q4_0) {
        const float d = half_at(scale, k);
        const uint4 q = *(const uint4 *)((const uint8_t *)codes + k * 16);
        const uint8_t *c = (const uint8_t *)&q;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = d * (float)((int)(c[i] & 15) - 8);
            x[16 + i] = d * (float)((int)(c[i] >> 4) - 8);
        }
    } else if (w_dt == DT_Q4_K) {
        // sub-block j of super-block sb: 6-bit scale and min from the 12
        // packed bytes; its codes are the low (j even) or high (j odd)
        // nibbles of code bytes 32 (j / 2) .. 32 (j / 2) + 31
        const int64_t sb = k >> 3;
        const int j = (int)(k & 7);
        const float d = half_at(scale, 2 * sb), dmin = half_at(scale, 2 * sb + 1);
        const uint8_t *s = sub + sb * 12;
        int sc, m;
        if (j < 4) {
            sc = s[j] & 63;
            m = s[j + 4] & 63;
        } else {
            sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
        const float d1 = d * (float)sc, m1 = dmin * (float)m;
        const uint4 *src = (const uint4 *)((const uint8_t *)codes + sb * 128 + (j >> 1) * 32);
        const uint4 q0 = src[0], q1 = src[1];
        const uint8_t *c0 = (const uint8_t *)&q0, *c1 = (const uint8_t *)&q1;
        const int sh = (j & 1) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = d1 * (float)((c0[i] >> sh) & 15) - m1;
            x[16 + i] = d1 * (float)((c1[i] >> sh) & 15) - m1;
        }
    } else {  // DT_Q6_K
        // unit j = 4 h + t of super-block sb covers weights 128 h + 32 t ..
        // +31: low 4 bits from the low (t < 2) or high nibble of low bytes
        // 64 h + 32 (t % 2) + l, high 2 bits from bits 2t, 2t+1 of high byte
        // 32 h + l; scales 8 h + 2 t (l < 16) and 8 h + 2 t + 1
        const int64_t sb = k >> 3;
        const int j = (int)(k & 7), h = j >> 2, t = j & 3;
        const float d = half_at(scale, sb);
        const int8_t *sc = (const int8_t *)sub + sb * 16 + 8 * h + 2 * t;
        const float d0 = d * (float)sc[0], d1 = d * (float)sc[1];
        const uint8_t *base = (const uint8_t *)codes + sb * 192;
        const uint4 *lo = (const uint4 *)(base + 64 * h + 32 * (t & 1));
        const uint4 *hi = (const uint4 *)(base + 128 + 32 * h);
        const uint4 l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
        const uint8_t *L0 = (const uint8_t *)&l0, *L1 = (const uint8_t *)&l1;
        const uint8_t *H0 = (const uint8_t *)&h0, *H1 = (const uint8_t *)&h1;
        const int lsh = (t >> 1) * 4, hsh = 2 * t;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int q0 = ((L0[i] >> lsh) & 15) | (((H0[i] >> hsh) & 3) << 4);
            const int q1 = ((L1[i] >> lsh) & 15) | (((H1[i] >> hsh) & 3) << 4);
            x[i] = d0 * (float)(q0 - 32);
            x[16 + i] = d1 * (float)(q1 - 32);
        }
    }
}

// dense storage widened to f32, one thread per element
__global__ void widen_kernel(int w_dt, const void *w, int64_t n, float *out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    float v;
    if (w_dt == DT_F16) v = to_f32(((const f16_t *)w)[idx]);
    else if (w_dt == DT_BF16) v = to_f32(((const bf16_t *)w)[idx]);
    else v = ((const float *)w)[idx];
    out[idx] = v;
}

// block formats to f32, one thread per unit of 32 weights
__global__ __launch_bounds__(256) void dequant_units_kernel(int w_dt, const void *codes, const uint16_t *scale,
                                                            const uint8_t *sub, int64_t units, float *out) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= units) return;
    float x[32];
    unit_values(w_dt, codes, scale, sub, k, x);
    float4 *dst = (float4 *)(out + k * 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) dst[c] = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
}

// Dense MFMA calibration: each wave runs `iters` rounds of 8 independent
// v_mfma_f32_32x32x16_bf16 chains on register operands (so the matrix core
// never waits on a result), then stores the sum of its accumulators so that
// nothing is optimised away.  32 * 32 * 16 * 2 flops per instruction.
// Operands (RND = false): small constant values, one A and one B register
// set, the same bits in every instruction.  RND = true: four A and four B
// sets of random bf16 values in [-1, 1) (a counter hash of thread, set and
// element), paired so that consecutive MFMAs differ in both operands, as
// they do in a GEMM.  The matrix core's power, and with it the clock the chip
// holds, depends on how many operand bits toggle, so the two rates differ.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return x;
}
template <bool RND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float *out) {
    constexpr int SETS = RND ? 4 : 1;
    bf16x8 a[SETS], b[SETS];
#pragma unroll
    for (int t = 0; t < SETS; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (RND) {
                const uint32_t h = probe_hash((blockIdx.x * 256 + threadIdx.x) * 64 + t * 8 + j);
                a[t][j] = (__bf16)((float)(h & 0xffff) * (1.f / 32768.f) - 1.f);
                b[t][j] = (__bf16)((float)(h >> 16) * (1.f / 32768.f) - 1.f);
            } else {
                a[t][j] = (__bf16)(1e-3f * (float)((threadIdx.x + j) & 7));
                b[t][j] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + j) & 7));
            }
        }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c)   // (a, b) sets (0,0) (1,1) (2,2) (3,3) (0,1) (1,2) (2,3) (3,0)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c % SETS], b[(c + c / 4) % SETS], acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// int8 MFMA calibration, and the cost of consuming it for block-scaled
// weights.  Each wave runs `iters` rounds of 4 independent
// v_mfma_i32_32x32x32_i8 (one 32-wide K block each, 65536 ops):
//   mode 0: the products accumulate in int32 (the plain int8 rate);
//   mode 1: every block's int32 result starts from zero and is folded into
//           f32 accumulators with a per-block scale for each of the lane's
//           16 rows (activations quantised per 32-block) times a per-block
//           scale for its column (the weight block's d): cvt, mul, fma per
//           element; the scales come from LDS, as they would in a GEMM;
//   mode 2: as mode 1 with one scale per activation row for all of K, so
//           only the column scale remains per block: cvt, fma per element.
typedef signed char i8x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Rescale chain c's block result t into facc (modes 1, 2); the scales of K
// block kb come from LDS.
template <int MODE>
__device__ __forceinline__ void i8_rescale(f32x16 &facc, const i32x16 &t, const float (*scales)[1024], int kb,
                                           int col, int g32) {
    const float sw = scales[1][kb * 32 + col];
    if constexpr (MODE == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 sa = *(const float4 *)&scales[0][kb * 32 + 8 * q + 4 * g32];
            const float s4[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[4 * q + r] = fmaf(s4[r] * sw, (float)t[4 * q + r], facc[4 * q + r]);
        }
    } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) facc[v] = fmaf(sw, (float)t[v], facc[v]);
    }
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_i8_probe_kernel(int iters, float *out) {
    __shared__ float scales[2][1024];
    for (int i = threadIdx.x; i < 2048; i += 256) scales[i >> 10][i & 1023] = 1e-3f * (float)((i * 37) & 63) + 1e-4f;
    __syncthreads();
    const int lane = threadIdx.x & 63, g32 = lane >> 5, col = lane & 31;
    i8x16 a, b[4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        a[j] = (signed char)(((threadIdx.x + j) & 15) - 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c][j] = (signed char)(((threadIdx.x * 3 + j + 5 * c) & 15) - 8);
    }
    i32x16 t[4];
    f32x16 facc[4];
    const i32x16 zero = {};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        t[c] = zero;
#pragma unroll
        for (int v = 0; v < 16; ++v) facc[c][v] = 0.f;
    }
    // The A operand passes through an empty asm statement once per round, so
    // that the compiler can neither hoist the rounds' identical products out
    // of the loop nor merge them; it emits no instruction.
    i32x4 ao = __builtin_bit_cast(i32x4, a);
    if constexpr (MODE == 0) {
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[c], t[c], 0, 0, 0);
    } else {
        // software-pipelined: block i of chain c is rescaled while the other
        // chains' MFMAs run, then chain c's next block is issued
#pragma unroll
        for (int c = 0; c < 4; ++c)
            t[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i8x16, ao), b[c], zero, 0, 0, 0);
        for (int i = 0; i < iters - 1; ++i) {
            asm volatile("" : "+v"(ao));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                i8_rescale<MODE>(facc[c], t[c], scales, (i * 4 + c) & 31, col, g32);
                t[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i8x16, ao), b[c], zero, 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            i8_rescale<MODE>(facc[c], t[c], scales, ((iters - 1) * 4 + c) & 31, col, g32);
            t[c] = zero;
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += facc[c][v] + (float)t[c][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Activations quantised per 32-block for the int8 path: one thread per
// block, 64 bytes in (4 x 16), 32 code bytes and one f32 scale out.
// d = max|x| / 127 and x / d are single correctly rounded f32 divisions (the
// default for '/' here), and roundf rounds halves away from zero.
template <typename T>
__global__ __launch_bounds__(256) void quant_act_kernel(const T *x, int64_t ldx, int64_t M, int64_t nb,
                                                        int8_t *q, int64_t ldq, float *d) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * nb) return;
    const int64_t m = i / nb, b = i - m * nb;
    const uint4 *src = (const uint4 *)(x + m * ldx + b * 32);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 w = src[c];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[8 * c + 2 * e] = to_f32(__builtin_bit_cast(T, (unsigned short)(u[e] & 0xffffu)));
            v[8 * c + 2 * e + 1] = to_f32(__builtin_bit_cast(T, (unsigned short)(u[e] >> 16)));
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const float dd = amax / 127.0f;
    uint32_t w[8];
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float r = dd == 0.f ? 0.f : fminf(fmaxf(roundf(v[4 * k4 + e] / dd), -127.f), 127.f);
            word |= ((uint32_t)(int)r & 0xffu) << (8 * e);
        }
        w[k4] = word;
    }
    uint4 *dst = (uint4 *)(q + m * ldq + b * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    d[m * nb + b] = dd;
}

// f32 values rounded to the act dtype, and a fill (graph-capturable, unlike
// a memset node)
template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(const float *x, int64_t n, T *y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = from_f32<T>(x[i]);
}

__global__ __launch_bounds__(256) void fill_kernel(float *x, int64_t n, float v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) x[i] = v;
}

// One thread per unit of 32 weights: the unit's codes and scales in, 64
// bytes of act values out.  Neighbouring threads take neighbouring units, so
// every wave reads and writes contiguous runs.
template <typename T>
__global__ __launch_bounds__(256) void expand_kernel(const ExpandJob *jobs, int njobs, int64_t nblk) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    int lo = 0, hi = njobs - 1;                  // the last job with blk0 <= b
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].blk0 <= b) lo = mid;
        else hi = mid - 1;
    }
    const ExpandJob j = jobs[lo];
    const int64_t k = b - j.blk0;
    float x[32];
    unit_values(j.w_dt, j.codes, j.scale, j.sub, k, x);
    uint4 *dst = (uint4 *)((T *)j.dst + k * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c)
        dst[c] = make_uint4(pack2<T>(x[8 * c], x[8 * c + 1]), pack2<T>(x[8 * c + 2], x[8 * c + 3]),
                            pack2<T>(x[8 * c + 4], x[8 * c + 5]), pack2<T>(x[8 * c + 6], x[8 * c + 7]));
}

}  // namespace

hipError_t launch_cast(const float *x, int64_t n, void *y, int y_dt, hipStream_t s) {
    if (n <= 0 || cdiv(n, 256) >= (1ll << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)cdiv(n, 256));
    switch (y_dt) {
        case DT_F32: hipLaunchKernelGGL(cast_kernel<float>, grid, dim3(256), 0, s, x, n, (float *)y); break;
        case DT_BF16: hipLaunchKernelGGL(cast_kernel<bf16_t>, grid, dim3(256), 0, s, x, n, (bf16_t *)y); break;
        case DT_F16: hipLaunchKernelGGL(cast_kernel<f16_t>, grid, dim3(256), 0, s, x, n, (f16_t *)y); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quant_act(int act_dt, const void *x, int64_t ldx, int64_t M, int64_t K, int8_t *q,
                            int64_t ldq, float *d, hipStream_t s) {
    // 16-byte rows of both sides: pitches and pointers
    if (M <= 0 || K <= 0 || K % 32 || ldx < K || ldq < K || ldq % 16 || ldx % 8 || ((uintptr_t)x & 15) ||
        ((uintptr_t)q & 15) || ((uintptr_t)d & 3))
        return hipErrorInvalidValue;
    const int64_t nb = K / 32, n = M * nb;
    if (cdiv(n, 256) >= (1ll << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)cdiv(n, 256));
    switch (act_dt) {
        case DT_BF16:
            hipLaunchKernelGGL(quant_act_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t *)x, ldx, M, nb, q, ldq, d);
            break;
        case DT_F16:
            hipLaunchKernelGGL(quant_act_kernel<f16_t>, grid, dim3(256), 0, s, (const f16_t *)x, ldx, M, nb, q, ldq, d);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mfma_probe(int workgroups, int iters, int operands, float *out, hipStream_t s) {
    if (workgroups <= 0 || iters <= 0 || operands < 0 || operands > 1 || !out) return hipErrorInvalidValue;
    if (operands == 0) hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(workgroups), dim3(256), 0, s, iters, out);
    else hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(workgroups), dim3(256), 0, s, iters, out);
    return hipGetLastError();
}

hipError_t launch_mfma_i8_probe(int workgroups, int iters, int mode, float *out, hipStream_t s) {
    if (workgroups <= 0 || iters <= 0 || mode < 0 || mode > 2 || !out) return hipErrorInvalidValue;
    if (mode == 0) hipLaunchKernelGGL(mfma_i8_probe_kernel<0>, dim3(workgroups), dim3(256), 0, s, iters, out);
    else if (mode == 1) hipLaunchKernelGGL(mfma_i8_probe_kernel<1>, dim3(workgroups), dim3(256), 0, s, iters, out);
    else hipLaunchKernelGGL(mfma_i8_probe_kernel<2>, dim3(workgroups), dim3(256), 0, s, iters, out);
    return hipGetLastError();
}

hipError_t launch_fill(float *x, int64_t n, float v, hipStream_t s) {
    if (n <= 0 || cdiv(n, 256) >= (1ll << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, x, n, v);
    return hipGetLastError();
}

hipError_t launch_expand(int act_dt, const ExpandJob *jobs, int njobs, int64_t nblk, hipStream_t s) {
    if (!jobs || njobs <= 0 || nblk <= 0 || cdiv(nblk, 256) >= (1ll << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)cdiv(nblk, 256));
    if (act_dt == DT_BF16) hipLaunchKernelGGL(expand_kernel<bf16_t>, grid, dim3(256), 0, s, jobs, njobs, nblk);
    else if (act_dt == DT_F16) hipLaunchKernelGGL(expand_kernel<f16_t>, grid, dim3(256), 0, s, jobs, njobs, nblk);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_patchify(int act_dt, const PatchifyArgs &a, hipStream_t s) {
    const int P = a.tubelet * a.patch * a.patch * 3;
    if (a.B <= 0 || a.patch <= 0 || a.tubelet <= 0 || a.H % a.patch || a.W % a.patch ||
        a.T % a.tubelet || a.ld < P)
        return hipErrorInvalidValue;
    const int64_t np = (int64_t)(a.T / a.tubelet) * (a.H / a.patch) * (a.W / a.patch);
    const int64_t total = (int64_t)a.B * np * a.ld;
    const dim3 grid((unsigned)cdiv(total, 256));
    switch (act_dt) {
        case DT_F32: hipLaunchKernelGGL(patchify_kernel<float>, grid, dim3(256), 0, s, a, total); break;
        case DT_BF16: hipLaunchKernelGGL(patchify_kernel<bf16_t>, grid, dim3(256), 0, s, a, total); break;
        case DT_F16: hipLaunchKernelGGL(patchify_kernel<f16_t>, grid, dim3(256), 0, s, a, total); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_layernorm(const float *x, int64_t rows, int dim, const float *gamma,
                            const float *beta, float eps, void *y, int y_dt, hipStream_t s) {
    if (rows <= 0 || dim % 64) return hipErrorInvalidValue;
    switch (y_dt) {
        case DT_F32: return ln_dispatch<float>(x, rows, dim, gamma, beta, eps, y, s);
        case DT_BF16: return ln_dispatch<bf16_t>(x, rows, dim, gamma, beta, eps, y, s);
        case DT_F16: return ln_dispatch<f16_t>(x, rows, dim, gamma, beta, eps, y, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cls_rows(float *x, const float *cls, const float *pos, int B, int N, int D,
                           hipStream_t s) {
    if (B <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cls_rows_kernel, dim3(B), dim3(256), 0, s, x, cls, pos, N, D);
    return hipGetLastError();
}

// out[i] = y[i] for n f32 values, 16 bytes per thread where both are aligned
__global__ __launch_bounds__(256) void copy_f32_kernel(const float *y, int64_t n, float *out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        ((float4 *)out)[i] = ((const float4 *)y)[i];
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = y[i];
}

hipError_t launch_copy_f32(const float *y, int64_t n, float *out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (((uintptr_t)y | (uintptr_t)out) & 15) return hipErrorInvalidValue;
    const int64_t blocks = std::min<int64_t>(cdiv(n / 4 + 1, 256), 4096);
    hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, y, n, out);
    return hipGetLastError();
}

hipError_t launch_pool_cls(const float *y, int B, int N, int D, float *out, hipStream_t s) {
    if (B <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pool_cls_kernel, dim3(B), dim3(256), 0, s, y, N, D, out);
    return hipGetLastError();
}

hipError_t launch_pool_mean(const float *y, int B, int N, int D, int first, float *part, float *out,
                            hipStream_t s) {
    if (B <= 0 || D % 64 || first >= N || !part) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pool_mean_part_kernel, dim3(B, D / 64, POOL_CHUNKS), dim3(256), 0, s, y, N, D, first, part);
    hipLaunchKernelGGL(pool_mean_fin_kernel, dim3((unsigned)cdiv((int64_t)B * D, 256)), dim3(256), 0, s, part, B, N,
                       D, first, out);
    return hipGetLastError();
}

hipError_t launch_dequant(int w_dt, const void *w, const uint16_t *scale, const uint8_t *sub, int64_t rows,
                          int64_t cols, float *out, hipStream_t s) {
    if (rows <= 0 || cols <= 0 || !w || !out) return hipErrorInvalidValue;
    const int64_t n = rows * cols;
    if (w_dt == DT_Q8_0 || w_dt == DT_Q4_0 || w_dt == DT_Q4_K || w_dt == DT_Q6_K) {
        const int64_t unit = (w_dt == DT_Q4_K || w_dt == DT_Q6_K) ? 256 : 32;
        if (cols % unit || !scale || ((w_dt == DT_Q4_K || w_dt == DT_Q6_K) && !sub)) return hipErrorInvalidValue;
        const int64_t units = n / 32;
        if (cdiv(units, 256) >= (1ll << 31)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(dequant_units_kernel, dim3((unsigned)cdiv(units, 256)), dim3(256), 0, s, w_dt, w, scale,
                           sub, units, out);
    } else if (w_dt == DT_F32 || w_dt == DT_F16 || w_dt == DT_BF16) {
        if (cdiv(n, 256) >= (1ll << 31)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(widen_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, w_dt, w, n, out);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace jepa
