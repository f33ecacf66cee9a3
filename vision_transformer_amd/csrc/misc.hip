// The bandwidth-bound kernels of the encoder: patchify (pixel ingest and
// normalisation), LayerNorm, CLS rows, pooling and dequantisation.
#include <algorithm>

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
    const float mean = wave_sum(s) * (1.f / D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float c = v[i] - mean;
        q = fmaf(c, c, q);
    }
    const float rs = rsqrtf(wave_sum(q) * (1.f / D) + eps);
    TO *yr = y + row * D;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int d = lane + 64 * i;
        yr[d] = from_f32<TO>((v[i] - mean) * rs * gam[d] + bet[d]);
    }
}

template <typename TO>
hipError_t ln_dispatch(const float *x, int64_t rows, int dim, const float *g, const float *b,
                       float eps, void *y, hipStream_t s) {
    dim3 grid((unsigned)cdiv(rows, 4));
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
// dequantisation to f32 (exact: f32(d) * integer code)
//   q8_0 packed: codes int8 [rows, cols], scales f16 [rows, cols/32]
//   q4_0 packed: blocks of 16 bytes [rows, cols/32], byte j = code j (low
//                nibble) | code j+16 (high nibble); scales as q8_0
// ---------------------------------------------------------------------------
__global__ void dequant_kernel(int w_dt, const void *w, const uint16_t *scale, int64_t rows,
                               int64_t cols, float *out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cols) return;
    const int64_t r = idx / cols, c = idx - r * cols;
    float v;
    if (w_dt == DT_Q8_0 || w_dt == DT_Q4_0) {
        const float d = (float)__builtin_bit_cast(_Float16, scale[r * (cols / 32) + c / 32]);
        int q;
        if (w_dt == DT_Q8_0) {
            q = ((const int8_t *)w)[idx];
        } else {
            const int e = (int)(c & 31);
            const uint8_t byte = ((const uint8_t *)w)[r * (cols / 2) + (c / 32) * 16 + (e & 15)];
            q = (e < 16 ? (byte & 15) : (byte >> 4)) - 8;
        }
        v = d * (float)q;
    } else if (w_dt == DT_F16) {
        v = to_f32(((const f16_t *)w)[idx]);
    } else if (w_dt == DT_BF16) {
        v = to_f32(((const bf16_t *)w)[idx]);
    } else {
        v = ((const float *)w)[idx];
    }
    out[idx] = v;
}

// Dense MFMA calibration: each wave runs `iters` rounds of 8 independent
// v_mfma_f32_32x32x16_bf16 chains on register operands (so the matrix core
// never waits on a result), then stores the sum of its accumulators so that
// nothing is optimised away.  32 * 32 * 16 * 2 flops per instruction.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float *out) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1e-3f * (float)((threadIdx.x + j) & 7));
        b[j] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + j) & 7));
    }
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[c][v];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
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

// One thread per block of 32 weights: 32 (q8_0) or 16 (q4_0) code bytes and
// the f16 scale in, 64 bytes of act values out.  Neighbouring threads take
// neighbouring blocks, so every wave reads and writes contiguous runs.
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
    const float d = (float)__builtin_bit_cast(_Float16, j.scale[k]);
    float x[32];
    if (j.w_dt == DT_Q8_0) {
        const uint4 *src = (const uint4 *)((const int8_t *)j.codes + k * 32);
        const uint4 q0 = src[0], q1 = src[1];
        const int8_t *c0 = (const int8_t *)&q0, *c1 = (const int8_t *)&q1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = d * (float)c0[i];
            x[16 + i] = d * (float)c1[i];
        }
    } else {
        const uint4 q = *(const uint4 *)((const uint8_t *)j.codes + k * 16);
        const uint8_t *c = (const uint8_t *)&q;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = d * (float)((int)(c[i] & 15) - 8);
            x[16 + i] = d * (float)((int)(c[i] >> 4) - 8);
        }
    }
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

hipError_t launch_mfma_probe(int workgroups, int iters, float *out, hipStream_t s) {
    if (workgroups <= 0 || iters <= 0 || !out) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, s, iters, out);
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

hipError_t launch_dequant(int w_dt, const void *w, const uint16_t *scale, int64_t rows,
                          int64_t cols, float *out, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipErrorInvalidValue;
    if ((w_dt == DT_Q8_0 || w_dt == DT_Q4_0) && (cols % 32 || !scale)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)cdiv(rows * cols, 256)), dim3(256), 0, s,
                       w_dt, w, scale, rows, cols, out);
    return hipGetLastError();
}

}  // namespace jepa
