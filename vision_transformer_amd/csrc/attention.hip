// Multi-head attention, head_dim 64, bidirectional or block-causal, as a
// flash-attention forward on MFMA: K and V tiles of 64 keys are staged in
// LDS, scores and probabilities stay in registers, softmax is online.
//
// Mask (LeVJEPA ViT-L/16 card, opening paragraph): under block-causal a
// patch token of temporal slot t attends to the patch tokens of slots <= t
// and not to CLS; CLS attends to every token.  With CLS as token 0 and
// tokens ordered slot by slot, every query's allowed keys form one range
// [lo, hi): lo = 1 (skip CLS) and hi = end of the query's slot.  Key tiles
// past the largest hi of a query tile are never visited (whole future-frame
// tiles skipped); a tile that straddles some query's hi masks elementwise.
// The CLS query of a block-causal item reads all N keys, so it runs in a
// separate small kernel rather than stretching the first query tile.
//
// Layout trick: each wave computes S^T = K Q^T (32 keys x 32 queries per
// MFMA), so lane l owns query l % 32 and holds 16 of its scores.  Those
// scores, exponentiated, are exactly the B operand of O^T = V^T P^T, so P
// never leaves registers.  V is written to LDS transposed, with the keys of
// each 32-key block permuted so that every lane's A operand is one
// contiguous LDS read.
#include "common.hpp"
#include "kernels.hpp"

namespace jepa {
namespace {

constexpr int DH = 64;      // head dim
constexpr int QT = 128;     // queries per workgroup (4 waves x 32)
constexpr int KT = 64;      // keys per step

// LDS column of key r (0..63 within a tile) in the transposed V tile: the
// k-slot that the P^T operand gives to that key.  Accumulator element v of
// lane group g holds key 8*(v/4) + 4*g + v%4 of its 32-key block; operand
// chunk c, slot j of group g takes element v = c*VEC + j.
template <int VEC, int KC>
__device__ __forceinline__ int vt_col(int r) {
    const int sb = r >> 5, kap = r & 31;
    const int g = (kap >> 2) & 1;
    const int v = 4 * (kap >> 3) + (kap & 3);
    return sb * 32 + (v / VEC) * KC + g * VEC + (v % VEC);
}

template <typename T>
__global__ __launch_bounds__(256, 2) void attn_kernel(const AttnArgs a, int q_start, int n_qtiles) {
    typedef Mfma<T> MM;
    constexpr int ES = sizeof(T);
    constexpr int VEC = MM::VEC, KC = MM::KC;
    constexpr int CE = 16 / ES;                 // elements per 16-byte chunk
    constexpr int KROWB = DH * ES + 16;         // K tile row bytes (padded)
    constexpr int VROWB = KT * ES + 16;         // V^T tile row bytes (padded)
    __shared__ __attribute__((aligned(16))) unsigned char sK[KT * KROWB];
    __shared__ __attribute__((aligned(16))) unsigned char sV[DH * VROWB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int b = blockIdx.z, h = blockIdx.y;
    const int tile = a.block_causal ? (n_qtiles - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int N = a.N, D = a.heads * DH;
    const int64_t ld = 3 * (int64_t)D;
    const T *base = (const T *)a.qkv + (int64_t)b * N * ld;
    const int q0 = q_start + tile * QT;
    const int qi = q0 + wave * 32 + (lane & 31);
    const bool qvalid = qi < N;

    // allowed key range of a query (see header)
    const int lo = (a.block_causal && a.has_cls) ? 1 : 0;
    auto hi_of = [&](int q) -> int {
        if (!a.block_causal || q >= N) return N;
        const int h_ = a.has_cls + a.per_slot * ((q - a.has_cls) / a.per_slot + 1);
        return h_ < N ? h_ : N;
    };
    const int my_hi = hi_of(qi);
    const int tile_last = (q0 + QT - 1 < N - 1) ? q0 + QT - 1 : N - 1;
    const int kend = hi_of(tile_last);
    const int hi_min = hi_of(q0);

    // Q operand, one 32-query column block per wave
    typename MM::vec qv[DH / KC];
#pragma unroll
    for (int c = 0; c < DH / KC; ++c) {
        if (qvalid)
            qv[c] = MM::load(base + (int64_t)qi * ld + h * DH + c * KC + g * VEC);
        else
            qv[c] = typename MM::vec{};
    }

    const float sl2 = 0.125f * 1.4426950408889634f;   // 1/sqrt(64) * log2(e)
    float m = -INFINITY, l = 0.f;
    f32x16 o[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) { o[0][v] = 0.f; o[1][v] = 0.f; }

    for (int k0 = lo; k0 < kend; k0 += KT) {
        __syncthreads();
        // stage K (row-major) and V (transposed, permuted) for keys k0..k0+63
        constexpr int CHUNKS = KT * DH / CE / 256;
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int ci = tid + 256 * i;
            const int r = ci / (DH / CE), c = ci % (DH / CE);
            const int key = k0 + r;
            uint4 kc = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
            if (key < N) {
                const T *row = base + (int64_t)key * ld + h * DH + c * CE;
                kc = *(const uint4 *)(row + D);
                vc = *(const uint4 *)(row + 2 * D);
            }
            *(uint4 *)(sK + r * KROWB + c * 16) = kc;
            const T *ve = (const T *)&vc;
            const int col = vt_col<VEC, KC>(r);
#pragma unroll
            for (int e = 0; e < CE; ++e) *(T *)(sV + (c * CE + e) * VROWB + col * ES) = ve[e];
        }
        __syncthreads();

        // S^T for the two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[sb][v] = 0.f;
#pragma unroll
            for (int c = 0; c < DH / KC; ++c) {
                typename MM::vec kv = MM::load(sK + (sb * 32 + (lane & 31)) * KROWB + (c * KC + g * VEC) * ES);
                s[sb] = MM::mma(kv, qv[c], s[sb]);
            }
        }
        if (k0 + KT > hi_min) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = k0 + sb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                    if (key >= my_hi) s[sb][v] = -INFINITY;
                }
        }
        // online softmax (row = this lane's query; its other half is lane ^ 32)
        float mt = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[sb][v]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m, mt);
        const float alpha = exp2f((m - mn) * sl2);
        const float mb = mn * sl2;
        m = mn;
        l *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) { o[0][v] *= alpha; o[1][v] *= alpha; }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2f(fmaf(s[sb][v], sl2, -mb));
                s[sb][v] = p;
                l += p;
            }
        // O^T += V^T P^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int cc = 0; cc < 32 / KC; ++cc) {
                float pv[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) pv[j] = s[sb][cc * VEC + j];
                typename MM::vec pb = pack_operand<T>(pv);
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    typename MM::vec va = MM::load(sV + (db * 32 + (lane & 31)) * VROWB +
                                                   (sb * 32 + cc * KC + g * VEC) * ES);
                    o[db] = MM::mma(va, pb, o[db]);
                }
            }
        }
    }

    l += __shfl_xor(l, 32, 64);
    if (!qvalid) return;
    const float inv = 1.f / l;
    T *out = (T *)a.out + ((int64_t)b * N + qi) * D + h * DH;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            out[db * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = from_f32<T>(o[db][v] * inv);
}

// The CLS query of a block-causal item: one workgroup per (head, item),
// scores for all N keys in LDS, then the weighted sum of V.
template <typename T>
__global__ __launch_bounds__(256) void attn_cls_kernel(const AttnArgs a) {
    extern __shared__ float sc[];                 // [N] scores, then probabilities
    __shared__ float qs[DH];
    __shared__ float red[256];
    const int tid = threadIdx.x;
    const int h = blockIdx.x, b = blockIdx.y;
    const int N = a.N, D = a.heads * DH;
    const int64_t ld = 3 * (int64_t)D;
    const T *base = (const T *)a.qkv + (int64_t)b * N * ld;
    if (tid < DH) qs[tid] = to_f32(base[h * DH + tid]);
    __syncthreads();
    float mx = -INFINITY;
    for (int j = tid; j < N; j += 256) {
        const T *k = base + (int64_t)j * ld + D + h * DH;
        float acc = 0.f;
#pragma unroll 8
        for (int d = 0; d < DH; ++d) acc = fmaf(qs[d], to_f32(k[d]), acc);
        acc *= 0.125f;
        sc[j] = acc;
        mx = fmaxf(mx, acc);
    }
    red[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float sum = 0.f;
    for (int j = tid; j < N; j += 256) {
        const float p = expf(sc[j] - mx);
        sc[j] = p;
        sum += p;
    }
    red[tid] = sum;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    sum = red[0];
    __syncthreads();
    const int d = tid & 63, part = tid >> 6;
    float acc = 0.f;
    for (int j = part; j < N; j += 4) acc = fmaf(sc[j], to_f32(base[(int64_t)j * ld + 2 * D + h * DH + d]), acc);
    red[tid] = acc;
    __syncthreads();
    if (tid < DH) {
        const float o = (red[tid] + red[tid + 64] + red[tid + 128] + red[tid + 192]) / sum;
        ((T *)a.out)[(int64_t)b * N * D + h * DH + tid] = from_f32<T>(o);
    }
}

template <typename T>
hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    const int q_start = (a.block_causal && a.has_cls) ? 1 : 0;
    const int n_q = a.N - q_start;
    const int n_qtiles = (int)cdiv(n_q, QT);
    if (n_qtiles > 0) {
        hipLaunchKernelGGL((attn_kernel<T>), dim3(n_qtiles, a.heads, a.B), dim3(256), 0, s, a,
                           q_start, n_qtiles);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (q_start) {
        hipLaunchKernelGGL((attn_cls_kernel<T>), dim3(a.heads, a.B), dim3(256),
                           (size_t)a.N * sizeof(float), s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

// Largest N whose scores fit the CLS kernel's dynamic LDS (kept under 64 KB).
constexpr int kMaxClsTokens = 15360;

hipError_t launch_attention(int act_dt, const AttnArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.N <= 0 || a.heads <= 0 || a.heads > 65535 || a.B > 65535)
        return hipErrorInvalidValue;
    if (a.block_causal && (a.per_slot <= 0 || (a.N - a.has_cls) % a.per_slot)) return hipErrorInvalidValue;
    if (a.block_causal && a.has_cls && a.N > kMaxClsTokens) return hipErrorInvalidValue;
    switch (act_dt) {
        case DT_F32: return launch_t<float>(a, s);
        case DT_BF16: return launch_t<bf16_t>(a, s);
        case DT_F16: return launch_t<f16_t>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace jepa
