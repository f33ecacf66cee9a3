// Multi-head attention, head_dim 64, bidirectional or block-causal, as a
// flash-attention forward on MFMA: K and V tiles of 64 keys are staged in
// LDS (double buffered, the next tile's loads in flight during the current
// tile's MFMAs), scores and probabilities stay in registers, softmax is
// online.
//
// Mask (LeVJEPA ViT-L/16 card, opening paragraph): under block-causal a
// patch token of temporal slot t attends to the patch tokens of slots <= t
// and not to CLS; CLS attends to every token.  With CLS as token 0 and
// tokens ordered slot by slot, every query's allowed keys form one range
// [lo, hi): lo = 1 (skip CLS) and hi = end of the query's slot.  Key tiles
// (aligned to multiples of 64) past the largest hi of a query tile are never
// visited, i.e. whole future-frame tiles are skipped; tiles that straddle a
// query's lo or hi mask elementwise.  The CLS query of a block-causal item
// reads all N keys: it rides along as an extra query slot (index N) of the
// last query tile, which visits every key anyway, with range [0, N).
//
// Layout: each wave computes S^T = K Q^T (32 keys x 32 queries per MFMA), so
// lane l owns query l % 32 and holds 16 of its scores; exponentiated, they
// are exactly the B operand of O^T = V^T P^T, so P never leaves registers.
// The A operand of that product is V^T, which the qkv GEMM writes once per
// head ([B, H, 64, npad]); a lane's 8 keys of one operand are two runs of 4
// keys (4g..4g+3 and 8+4g..8+4g+3 of a 16-key group), which V^T stores
// side by side (vt_pos), so the operand is one 16-byte LDS read.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace jepa {
namespace {

constexpr int QT = 128;     // queries per workgroup (4 waves x 32)
constexpr int KT = 64;      // keys per step
constexpr int ATTN_QB2_MIN_N = 4096;   // 16-bit, bidirectional, head dim 64: 64 queries per wave from here

template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void attn_kernel(const AttnArgs a, int q_start, int n_qtiles) {
    typedef Mfma<T> MM;
    constexpr int ES = sizeof(T);
    constexpr int VEC = MM::VEC, KC = MM::KC;
    constexpr int CE = 16 / ES;                 // elements per 16-byte chunk
    constexpr int ROWK = DH * ES + 16;          // LDS bytes of a K row (DH elements + pad)
    constexpr int ROWV = 64 * ES + 16;          // LDS bytes of a V^T row (64 keys + pad)
    constexpr int KCH = DH / CE, VCH = 64 / CE; // 16-byte chunks per K row, per V^T row
    constexpr int KCHUNKS = 64 * KCH / 256, VCHUNKS = DH * VCH / 256;   // per thread
    static_assert(KCHUNKS >= 1 && VCHUNKS >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) unsigned char sK[2][64 * ROWK];
    __shared__ __attribute__((aligned(16))) unsigned char sV[2][DH * ROWV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    // grid (head, item, query tile): with the head fastest, all query tiles of
    // one (item, head) land on the same XCD under round-robin dispatch (when
    // heads is a multiple of 8) and share its L2; block-causal tiles go
    // heaviest (latest slot) first
    const int h = blockIdx.x, b = blockIdx.y;
    // blockIdx.z = query tile * S + key split (S = a.kvsplit, 1: no split)
    const int S = a.kvsplit > 1 ? a.kvsplit : 1;
    const int zq = (int)blockIdx.z / S, split = (int)blockIdx.z % S;
    const int tile = a.block_causal ? (n_qtiles - 1 - zq) : zq;
    const int N = a.N, D = a.heads * DH;
    const T *qk = (const T *)a.qk + (int64_t)b * N * a.ld_qk;
    const T *vt = (const T *)a.vt + ((int64_t)b * a.heads + h) * DH * a.npad;
    const int q0 = q_start + tile * QT;
    const int qi = q0 + wave * 32 + (lane & 31);
    // allowed key range of a query (see header); slot N is the CLS query
    const int lo = (a.block_causal && a.has_cls) ? 1 : 0;
    const bool cls_lane = lo && qi == N;
    const bool qvalid = qi < N || cls_lane;
    const int qrow = cls_lane ? 0 : qi;
    const int my_lo = cls_lane ? 0 : lo;
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
            qv[c] = MM::load(qk + (int64_t)qrow * a.ld_qk + h * DH + c * KC + g * VEC);
        else
            qv[c] = typename MM::vec{};
    }

    // ---- K / V^T tile staging: registers -> LDS ----
    uint4 kreg[KCHUNKS], vreg[VCHUNKS];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KCHUNKS; ++i) {
            const int ci = tid + 256 * i;
            const int r = ci / KCH, c = ci % KCH;
            const int key = k0 + r;
            kreg[i] = make_uint4(0, 0, 0, 0);
            if (key < N) kreg[i] = *(const uint4 *)(qk + (int64_t)key * a.ld_qk + D + h * DH + c * CE);
        }
#pragma unroll
        for (int i = 0; i < VCHUNKS; ++i) {
            // V^T row r (= dim d), keys k0 + c*CE .. ; npad covers the tile
            const int ci = tid + 256 * i;
            const int r = ci / VCH, c = ci % VCH;
            vreg[i] = *(const uint4 *)(vt + (int64_t)r * a.npad + k0 + c * CE);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCHUNKS; ++i) {
            const int ci = tid + 256 * i;
            *(uint4 *)(sK[buf] + (ci / KCH) * ROWK + (ci % KCH) * 16) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VCHUNKS; ++i) {
            const int ci = tid + 256 * i;
            *(uint4 *)(sV[buf] + (ci / VCH) * ROWV + (ci % VCH) * 16) = vreg[i];
        }
    };

    const float sl2 = a.q_prescaled ? 1.f : attn_q_scale(DH);   // score -> base-2 exponent
    float m = -INFINITY, l = 0.f;
    constexpr int NDB = DH / 32;                 // 32-dim blocks of the output
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = 0.f;

    // this split's key tiles: [kb0, ke) of the query tile's [kbeg, kend)
    const int kbeg = lo & ~(KT - 1);
    const int nt = (kend - kbeg + KT - 1) / KT, per = (nt + S - 1) / S;
    const int kb0 = kbeg + split * per * KT, ke = min(kend, kb0 + per * KT);
    if (kb0 < ke) {
    load_tile(kb0);
    store_tile(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kb0; k0 < ke; k0 += KT, buf ^= 1) {
        const bool more = k0 + KT < ke;
        if (more) load_tile(k0 + KT);
        const unsigned char *kb = sK[buf];
        const unsigned char *vb = sV[buf];

        // S^T for the two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[sb][v] = 0.f;
#pragma unroll
            for (int c = 0; c < DH / KC; ++c) {
                typename MM::vec kv = MM::load(kb + (sb * 32 + (lane & 31)) * ROWK + (c * KC + g * VEC) * ES);
                s[sb] = MM::mma(kv, qv[c], s[sb]);
            }
        }
        if (k0 < lo || k0 + KT > hi_min) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = k0 + sb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                    if (key < my_lo || key >= my_hi) s[sb][v] = -INFINITY;
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
        if (__any(mn > m)) {          // rescale only when some running max grew
            // (a lane whose max is still -inf has o = l = 0: alpha 0, not the
            // NaN of -inf - -inf)
            const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * sl2);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
            m = mn;
        }
        // (a query with no allowed key yet, possible in a key split, keeps
        // m = -inf and p = 0)
        const float mb = m == -INFINITY ? 0.f : m * sl2;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[sb][v], sl2, -mb));
                s[sb][v] = p;
                l += p;
            }
        // O^T += V^T P^T: operand chunk cc, slot j of lane group g is key
        // 8*(v/4) + 4*g + v%4 of the 32-key block, v = cc*VEC + j
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int cc = 0; cc < 32 / KC; ++cc) {
                float pv[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) pv[j] = s[sb][cc * VEC + j];
                typename MM::vec pb = pack_operand<T>(pv);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const unsigned char *row = vb + (db * 32 + (lane & 31)) * ROWV;
                    typename MM::vec va;
                    if constexpr (VEC == 8) {
                        // keys 16*cc + 4*g + {0-3, 8-11}: 16 contiguous bytes at their V^T position
                        va = MM::load(row + (sb * 32 + 16 * cc + 8 * g) * ES);
                    } else {
                        const int k = sb * 32 + 8 * (cc >> 2) + 4 * g + (cc & 3);
                        va = MM::load(row + vt_pos(k) * ES);
                    }
                    o[db] = MM::mma(va, pb, o[db]);
                }
            }
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }
    }

    l += __shfl_xor(l, 32, 64);
    if (!qvalid) return;
    if (S > 1) {
        // unnormalised output, running max (score units) and sum of this
        // split, row ((split*B + b)*heads + h)*N + qrow of the scratch
        float *pr = a.kvpart + ((((int64_t)split * a.B + b) * a.heads + h) * N + qrow) * (DH + 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) pr[db * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = o[db][v];
        if (g == 0) {
            pr[DH] = m;
            pr[DH + 1] = l;
        }
        return;
    }
    const float inv = 1.f / l;
    T *out = (T *)a.out + ((int64_t)b * N + qrow) * D + h * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            out[db * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = from_f32<T>(o[db][v] * inv);
}

// 16-bit variant: K and V^T tiles go global -> LDS directly
// (global_load_lds_dwordx4, lane i of a wave instruction lands at base + 16 i)
// into unpadded 128-byte rows whose 16-byte chunks are XOR-swizzled (chunk c
// of row r in slot c ^ swz(r)), two stages.  Each step reads all of its
// tile's MFMA operands out of LDS into registers first and only then issues
// the next tile's loads, so no LDS read follows a load in flight: the loads
// overlap the step's whole MFMA + softmax time.  No staging registers for
// the loads, no LDS write instructions.
// depends on row bits 0-4 only, so rows r and r + 32 share it
__device__ __forceinline__ int aswz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// The smallest value of the 16-bit type T that is >= x (x finite).
template <typename T> __device__ __forceinline__ float round_up_t(float x);
template <> __device__ __forceinline__ float round_up_t<bf16_t>(float x) {
    uint32_t u = __float_as_uint(x);
    u = (int32_t)u >= 0 ? (u + 0xFFFFu) & 0xFFFF0000u : u & 0xFFFF0000u;   // magnitude up if x >= 0, else down
    return __uint_as_float(u);
}
template <> __device__ __forceinline__ float round_up_t<f16_t>(float x) {
    _Float16 h = (_Float16)x;
    if ((float)h < x) {
        uint16_t b = __builtin_bit_cast(uint16_t, h);
        b = (b & 0x8000) ? b - 1 : b + 1;                                       // one step up
        h = __builtin_bit_cast(_Float16, b);
    }
    return (float)h;
}

// QS: the q columns hold q * ATTN_Q_SCALE, so q.k is the base-2 exponent,
// and the reference max m enters S through the MFMA itself: an extra 8-deep
// k chunk where K contributes 1 at dimension 64 and Q contributes -m (m kept
// exactly representable in T).  S then comes out as the exponent s - m and
// p = exp2(S) needs no VALU arithmetic before the exponential.
// QB query blocks of 32 per wave (QB = 2: 64 queries, 256 per workgroup).
// Every K and V^T operand a wave reads from LDS then feeds QB MFMAs, so the
// LDS read traffic per flop is 1/QB of one block's.  With one block per wave
// the LDS read bursts after each tile's barrier, four waves per SIMD, cap
// the MFMA rate well below its peak.
template <typename T, bool QS, int DH, int QB>
__global__ __launch_bounds__(256, QB == 1 ? 3 : 2) void attn16_kernel(const AttnArgs a, int q_start, int n_qtiles) {
    typedef Mfma<T> MM;
    typedef typename MM::vec vec;
    static_assert(sizeof(T) == 2, "16-bit operands");
    static_assert(DH == 32 || DH == 64, "head dims built");
    static_assert(QB == 1 || QB == 2, "query blocks per wave");
    constexpr int WQ = 32 * QB;                  // queries per wave
    constexpr int QTW = 4 * WQ;                  // queries per workgroup
    constexpr int RK = DH * 2;                   // bytes of a K row in LDS (unpadded)
    constexpr int CK = RK / 16;                  // its 16-byte chunks: 4 or 8
    constexpr int TBK = 64 * RK, TBV = DH * 128; // bytes of a K tile (64 keys) and a V^T tile
    constexpr int NI = DH / 32;                  // load instructions per operand per thread
    constexpr int NDB = DH / 32;                 // 32-dim blocks of the output
    // one array per stage: the compiler gives each its own alias scope, so
    // reads of one stage need not wait for loads landing in the other
    __shared__ __attribute__((aligned(1024))) unsigned char sK0[TBK];
    __shared__ __attribute__((aligned(1024))) unsigned char sK1[TBK];
    __shared__ __attribute__((aligned(1024))) unsigned char sV0[TBV];
    __shared__ __attribute__((aligned(1024))) unsigned char sV1[TBV];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS-load bases in SGPRs
    const int h = blockIdx.x, b = blockIdx.y;
    const int tile = a.block_causal ? (n_qtiles - 1 - (int)blockIdx.z) : (int)blockIdx.z;
    const int N = a.N, D = a.heads * DH;
    const T *qk = (const T *)a.qk + (int64_t)b * N * a.ld_qk;
    const T *vt = (const T *)a.vt + ((int64_t)b * a.heads + h) * DH * a.npad;
    const int q0 = q_start + tile * QTW;
    const int qw = q0 + wave * WQ;               // the wave's first query slot
    // allowed key range of a query (see header); slot N is the CLS query
    const int lo = (a.block_causal && a.has_cls) ? 1 : 0;
    auto hi_of = [&](int q) -> int {
        if (!a.block_causal || q >= N) return N;
        const int h_ = a.has_cls + a.per_slot * ((q - a.has_cls) / a.per_slot + 1);
        return h_ < N ? h_ : N;
    };
    // this lane's query of each block
    bool qvalid[QB];
    int qrow[QB], my_lo[QB], my_hi[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + qb * 32 + (lane & 31);
        const bool cls_lane = lo && qi == N;
        qvalid[qb] = qi < N || cls_lane;
        qrow[qb] = cls_lane ? 0 : qi;
        my_lo[qb] = cls_lane ? 0 : lo;
        my_hi[qb] = hi_of(qi);
    }
    const int tile_last = (q0 + QTW - 1 < N - 1) ? q0 + QTW - 1 : N - 1;
    const int kend = hi_of(tile_last);
    const int hi_min = hi_of(qw);                // this wave's queries: the smallest end
    // and the largest (its last slot, or the CLS slot N); key tiles at or past
    // it are masked for every lane of the wave, whose step then skips its
    // MFMAs and softmax (p would be exactly 0) but still loads and syncs
    const int w_end = hi_of(min(qw + WQ - 1, N));
    const int kbeg = lo & ~(KT - 1);
    const int ntiles = (kend - kbeg + KT - 1) / KT;

    vec qv[QB][DH / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int c = 0; c < DH / 16; ++c)
            qv[qb][c] = qvalid[qb] ? MM::load(qk + (int64_t)qrow[qb] * a.ld_qk + h * DH + c * 16 + g * 8) : vec{};

    // This thread's chunks of each tile: chunk id ci = i*256 + tid; a K row
    // has CK chunks (row ci / CK, slot ci % CK), a V^T row 8 (row ci >> 3,
    // slot ci & 7); a slot holds global chunk slot ^ swz(row).  Loads go
    // through buffer resources over the item's K rows and the (item, head)'s
    // V^T rows: the thread's byte offsets are fixed and a tile adds a uniform
    // one; key rows past the item's N read as 0 (masked keys).  Chunk i = 1
    // (head dim 64) is chunk 0's, 32 rows on (same swizzle): a uniform offset.
    uint32_t koffg, voffg;
    {
        const int rk = tid / CK, rv = tid >> 3;
        const int colk = ((tid % CK) ^ (aswz(rk) & (CK - 1))) * 8;   // element offsets of the chunks
        const int colv = ((tid & 7) ^ aswz(rv)) * 8;
        koffg = (uint32_t)((rk * a.ld_qk + colk) * (int64_t)sizeof(T));
        voffg = (uint32_t)((rv * a.npad + colv) * (int64_t)sizeof(T));
    }
    const uint32_t k32 = (uint32_t)(32 * a.ld_qk * (int64_t)sizeof(T)), v32 = (uint32_t)(32 * a.npad * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(qk + D + h * DH), 0, (int)(((int64_t)N * a.ld_qk - D - h * DH) * (int64_t)sizeof(T)), 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vt, 0, (int)((int64_t)DH * a.npad * (int64_t)sizeof(T)), 0x00020000);
    auto issue = [&](int t, auto ST) __attribute__((always_inline)) {
        unsigned char *sk = decltype(ST)::value ? sK1 : sK0;
        unsigned char *sv = decltype(ST)::value ? sV1 : sV0;
        const int k0 = kbeg + t * KT;
        const uint32_t ks = (uint32_t)(k0 * a.ld_qk * (int64_t)sizeof(T)), vs = (uint32_t)(k0 * sizeof(T));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int base = (i * 256 + wave * 64) * 16;  // LDS byte offset of lane 0
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void *)(sk + base),
                                                     16, koffg, ks + i * k32, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void *)(sv + base),
                                                     16, voffg, vs + i * v32, 0, 0);
        }
    };

    const float sl2 = QS ? 1.f : attn_q_scale(DH);   // score -> base-2 exponent
    // The running max m is a reference, not the exact max: it is raised only
    // when a score exceeds it by TH (2^8 in p), so p <= 2^8 and the rescale of
    // O and l runs a few times per query instead of at most tiles.  Any
    // reference gives the same softmax once O is divided by l.
    const float TH = 8.f / sl2;
    float m[QB], l0[QB], l1[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { m[qb] = QS ? 0.f : -INFINITY; l0[qb] = 0.f; l1[qb] = 0.f; }
    bool first = true;
    // QS: the extra k chunk's operands (dimension 64 of K is 1, of Q is -m),
    // for the 8-deep MFMA (4 elements per lane: half the registers and cycles
    // of a 16-deep chunk)
    typedef typename std::conditional<std::is_same<T, bf16_t>::value, __bf16, _Float16>::type elem_t;
    typedef elem_t x4 __attribute__((ext_vector_type(4)));
    x4 kx{}, qx[QB];
    kx[0] = g == 0 ? (elem_t)1.f : (elem_t)0.f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qx[qb] = x4{};
    auto mma_x = [&](const x4 &q_x, const f32x16 &c) __attribute__((always_inline)) -> f32x16 {
        if constexpr (std::is_same<T, bf16_t>::value) {
            typedef short s4 __attribute__((ext_vector_type(4)));
            return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s4, kx), __builtin_bit_cast(s4, q_x), c, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x8f16(kx, q_x, c, 0, 0, 0);
        }
    };
    f32x16 o[QB][NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[qb][db][v] = 0.f;

    const int r0 = lane & 31, sw = aswz(r0);
    // this lane's LDS byte offsets of the tile's operands in rows 0..31; the
    // second 32-row block (same swizzle) and the stage add constants
    int koff[DH / 16], voff[4];
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) koff[c] = r0 * RK + (((2 * c + g) ^ (sw & (CK - 1))) << 4);
    // V^T operand of 16-key group kg: keys 16*kg + 8*(j/4) + 4*g + j%4,
    // stored contiguously as chunk 2*kg + g of the row
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) voff[kg] = r0 * 128 + (((2 * kg + g) ^ sw) << 4);
    // row sums from the packed P operand (the values PV multiplies): two
    // products of (p, 1) per instruction, two chains
    const uint32_t ones = sizeof(T) == 2 && std::is_same<T, bf16_t>::value ? 0x3f803f80u : 0x3c003c00u;
    auto rowsum = [&](const vec &pb, float &s0, float &s1) __attribute__((always_inline)) {
        const uint4 w = __builtin_bit_cast(uint4, pb);
        if constexpr (std::is_same<T, bf16_t>::value) {
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            const b2 one = __builtin_bit_cast(b2, ones);
            s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w.x), one, s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w.y), one, s1, false);
            s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w.z), one, s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w.w), one, s1, false);
        } else {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            const h2 one = __builtin_bit_cast(h2, ones);
            s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w.x), one, s0, false);
            s1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w.y), one, s1, false);
            s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w.z), one, s0, false);
            s1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w.w), one, s1, false);
        }
    };

    // Tile t in stage ST: the next tile's loads issued into the other stage,
    // S = K Q^T from K operands read block by block (each feeding every query
    // block), the softmax per query block, then the V operands (read only
    // now, so K's and V's registers are never live together), each feeding
    // O^T += V^T P^T of every query block.
    auto step = [&](auto ST, int t) __attribute__((always_inline)) {
        constexpr int st = decltype(ST)::value;
        const unsigned char *sk = st ? sK1 : sK0;
        const unsigned char *sv = st ? sV1 : sV0;
        __builtin_amdgcn_s_waitcnt(0xF70);     // vmcnt(0): this wave's loads of tile t landed
        __builtin_amdgcn_s_barrier();           // everyone's did; everyone is done with the other stage
        if (t + 1 < ntiles) issue(t + 1, std::integral_constant<int, st ^ 1>{});

        // S^T = K Q^T, one 32-key block at a time
        const int k0 = kbeg + t * KT;
        if (k0 >= w_end) return;
        f32x16 s[QB][2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            vec kf[DH / 16];
#pragma unroll
            for (int c = 0; c < DH / 16; ++c) kf[c] = MM::load(sk + sb * 32 * RK + koff[c]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) s[qb][sb][v] = 0.f;
#pragma unroll
                for (int c = 0; c < DH / 16; ++c) s[qb][sb] = MM::mma(kf[c], qv[qb][c], s[qb][sb]);
                if constexpr (QS) s[qb][sb] = mma_x(qx[qb], s[qb][sb]);   // - m
            }
        }
        // masks, in float arithmetic (no per-element lane masks to hold):
        // the lane's keys are k0 + 4g + off, off = sb*32 + 8*(v/4) + v%4;
        // key < lo happens only for the CLS key 0 (lo = 1, first tile)
        if (k0 < lo) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                if (g == 0 && my_lo[qb] > 0) s[qb][0][0] = -INFINITY;
        }
        if (k0 + KT > hi_min) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // key < hi  <=>  (hi - k0 - 4g) - 0.5 - off > 0; times +inf that
                // is +inf (keep) or -inf (mask), never 0 * inf
                const float ch = (float)(my_hi[qb] - k0 - 4 * g) - 0.5f;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float off = (float)(sb * 32 + 8 * (v >> 2) + (v & 3));
                        s[qb][sb][v] = fminf(s[qb][sb][v], (ch - off) * INFINITY);
                    }
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // the max of this lane's half of its query's scores (the other
            // half is in lane ^ 32), as two independent chains
            float mh[2] = {-INFINITY, -INFINITY};
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mh[sb] = fmaxf(mh[sb], s[qb][sb][v]);
            float mt = fmaxf(mh[0], mh[1]);
            // A query's max passes a bound iff one of its halves does, and
            // the tests below are over the whole wave, so the halves are
            // combined (a cross-lane exchange) only when the reference moves.
            if constexpr (QS) {
                // s already holds the exponent relative to m; the first tile
                // sets m (its max rounded up to T), later ones raise it past TH
                if (first || __any(mt > TH)) {
                    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                    const float mn = (first || mt > 0.f) ? round_up_t<T>(m[qb] + mt) : m[qb];
                    const float d = mn - m[qb];
                    if (!first) {
                        const float alpha = __builtin_amdgcn_exp2f(-d);
                        l0[qb] *= alpha;
                        l1[qb] *= alpha;
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
#pragma unroll
                            for (int v = 0; v < 16; ++v) o[qb][db][v] *= alpha;
                    }
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                        for (int v = 0; v < 16; ++v) s[qb][sb][v] -= d;
                    m[qb] = mn;
                    qx[qb][0] = g == 0 ? (elem_t)(-mn) : (elem_t)0.f;
                }
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) s[qb][sb][v] = __builtin_amdgcn_exp2f(s[qb][sb][v]);
            } else {
                if (__any(mt > m[qb] + TH)) {
                    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                    const float mn = fmaxf(m[qb], mt);
                    const float alpha = __builtin_amdgcn_exp2f((m[qb] - mn) * sl2);
                    l0[qb] *= alpha;
                    l1[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int v = 0; v < 16; ++v) o[qb][db][v] *= alpha;
                    m[qb] = mn;
                }
                const float mb = m[qb] * sl2;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) s[qb][sb][v] = __builtin_amdgcn_exp2f(fmaf(s[qb][sb][v], sl2, -mb));
            }
        }
        first = false;
        // O^T += V^T P^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                vec pb[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float pv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) pv[j] = s[qb][sb][cc * 8 + j];
                    pb[qb] = pack_operand<T>(pv);
                    rowsum(pb[qb], l0[qb], l1[qb]);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const vec vop = MM::load(sv + db * 4096 + voff[2 * sb + cc]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[qb][db] = MM::mma(vop, pb[qb], o[qb][db]);
                }
            }
    };

    issue(0, std::integral_constant<int, 0>{});
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < ntiles) step(std::integral_constant<int, 0>{}, t);

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float l = l0[qb] + l1[qb];
        l += __shfl_xor(l, 32, 64);
        if (!qvalid[qb]) continue;
        const float inv = 1.f / l;
        T *out = (T *)a.out + ((int64_t)b * N + qrow[qb]) * D + h * DH;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                out[db * 32 + 8 * (v >> 2) + 4 * g + (v & 3)] = from_f32<T>(o[qb][db][v] * inv);
    }
}

// Merge of the key splits of the f32 kernel: per output row and column, the
// splits' outputs and sums weighted by exp2((m_s - max m) * sl2), in split
// order.
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *part, int S, int B, int heads, int N, float sl2,
                                                         T *out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)B * heads * N;
    if (i >= rows * DH) return;
    const int64_t r = i / DH, d = i - r * DH;            // r = (b*heads + h)*N + q
    const int64_t q = r % N, bh = r / N, h = bh % heads, b = bh / heads;
    float mx = -INFINITY;
    for (int z = 0; z < S; ++z) mx = fmaxf(mx, part[(z * rows + r) * (DH + 2) + DH]);
    float num = 0.f, den = 0.f;
    for (int z = 0; z < S; ++z) {
        const float *pz = part + (z * rows + r) * (DH + 2);
        const float w = __builtin_amdgcn_exp2f((pz[DH] - mx) * sl2);
        num += w * pz[d];
        den += w * pz[DH + 1];
    }
    out[(b * N + q) * (int64_t)heads * DH + h * DH + d] = from_f32<T>(num / den);
}

// One query row per item against that item's N keys and values (the
// classifier head's cross-attention), one workgroup per (head, item).  The
// scores go to LDS (one key per thread per pass, 16-byte key loads), then
// their max, the exponentials and their sum; the output is the weighted sum
// of the value rows, DH columns by 256/DH key phases, reduced in LDS.  f32
// arithmetic; the kernel reads K and V once and is bound by that.
template <typename T, int DH>
__global__ __launch_bounds__(256) void xattn_kernel(const T *q, const T *k, const T *v, int64_t ldkv, int N,
                                                    int heads, T *out) {
    constexpr int CE = 16 / (int)sizeof(T);     // elements per 16-byte load
    constexpr int PH = 256 / DH;                // key phases of the value pass
    constexpr float SC = DH == 32 ? 0.17677669529663687f : 0.125f;   // 1 / sqrt(DH)
    __shared__ float sp[XATTN_MAX_N];
    __shared__ float sq[DH];
    __shared__ float red[256];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t D = (int64_t)heads * DH;
    if (tid < DH) sq[tid] = to_f32(q[b * D + h * DH + tid]) * SC;
    __syncthreads();
    const T *kb = k + (int64_t)b * N * ldkv + h * DH;
    float mx = -INFINITY;
    for (int n = tid; n < N; n += 256) {
        const uint4 *kr = (const uint4 *)(kb + (int64_t)n * ldkv);
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < DH / CE; ++c) {
            const uint4 w = kr[c];
            const T *e = (const T *)&w;
#pragma unroll
            for (int j = 0; j < CE; ++j) s = fmaf(sq[c * CE + j], to_f32(e[j]), s);
        }
        sp[n] = s;
        mx = fmaxf(mx, s);
    }
    red[tid] = mx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float sum = 0.f;
    for (int n = tid; n < N; n += 256) {
        const float p = __expf(sp[n] - mx);
        sp[n] = p;
        sum += p;
    }
    red[tid] = sum;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    sum = red[0];
    __syncthreads();
    const int c = tid % DH, ph = tid / DH;
    const T *vb = v + (int64_t)b * N * ldkv + h * DH + c;
    float acc = 0.f;
    for (int n = ph; n < N; n += PH) acc = fmaf(sp[n], to_f32(vb[(int64_t)n * ldkv]), acc);
    red[tid] = acc;
    __syncthreads();
    if (tid < DH) {
        float o = 0.f;
        for (int p = 0; p < PH; ++p) o += red[p * DH + tid];
        out[b * D + h * DH + tid] = from_f32<T>(o / sum);
    }
}

// v columns of qkv [B*N, 3D] -> vt [B, D, npad] (row = v column, i.e. head
// h's dims at rows h*dh..), token n at vt_pos(n) (positions of no token
// untouched); blockIdx.y picks a group of 64 v columns
template <typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T *qkv, int N, int D, T *vt,
                                                          int64_t npad) {
    __shared__ T tile[64][65];
    const int b = blockIdx.z, c0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int n = n0 + r;
        if (n < N) tile[r][tx] = qkv[((int64_t)b * N + n) * 3 * D + 2 * D + c0 + tx];
    }
    __syncthreads();
    for (int d = ty; d < 64; d += 4) {
        const int n = n0 + tx;
        if (n < N) vt[((int64_t)b * D + c0 + d) * npad + vt_pos(n)] = tile[tx][d];
    }
}

template <typename T, int DH>
hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    // block-causal with CLS: query tiles cover tokens 1..N-1 plus the CLS
    // slot N, i.e. N slots from 1; otherwise tokens 0..N-1
    const int q_start = (a.block_causal && a.has_cls) ? 1 : 0;
    const int n_qtiles = (int)cdiv(a.N, QT);
    if (n_qtiles > 0) {
        const dim3 grid(a.heads, a.B, n_qtiles);
        if constexpr (sizeof(T) == 2) {
            // 64 queries per wave (256 per workgroup) for long bidirectional
            // head-64 sequences, where halving the LDS operand reads per flop
            // measured faster (8192 tokens: 310 vs 320-328 us); 32 per wave
            // elsewhere (block-causal 3137 tokens: 106 vs 121 us; 2048
            // tokens: even; head dim 32: 173 vs 191 us)
            if (!a.block_causal && DH == 64 && a.N >= ATTN_QB2_MIN_N) {
                const int nq2 = (int)cdiv(a.N, 2 * QT);
                const dim3 grid2(a.heads, a.B, nq2);
                if (a.q_prescaled)
                    hipLaunchKernelGGL((attn16_kernel<T, true, DH, 2>), grid2, dim3(256), 0, s, a, q_start, nq2);
                else
                    hipLaunchKernelGGL((attn16_kernel<T, false, DH, 2>), grid2, dim3(256), 0, s, a, q_start, nq2);
            } else if (a.q_prescaled) {
                hipLaunchKernelGGL((attn16_kernel<T, true, DH, 1>), grid, dim3(256), 0, s, a, q_start, n_qtiles);
            } else {
                hipLaunchKernelGGL((attn16_kernel<T, false, DH, 1>), grid, dim3(256), 0, s, a, q_start, n_qtiles);
            }
        } else {
            // few workgroups (small f32 models): split each query tile's keys
            // over S workgroups and merge the splits in a second pass
            const int64_t wgs = (int64_t)a.heads * a.B * n_qtiles;
            const int kt = (int)cdiv(a.N + 1, KT);
            const int S = (a.kvpart && 2 * wgs < 256 && kt >= 2) ? (kt < KVSPLIT_MAX ? kt : KVSPLIT_MAX) : 1;
            if (S > 1 && (int64_t)n_qtiles * S < 65535) {
                AttnArgs as = a;
                as.kvsplit = S;
                hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(a.heads, a.B, n_qtiles * S), dim3(256), 0, s, as,
                                   q_start, n_qtiles);
                const int64_t n = (int64_t)a.B * a.heads * a.N * DH;
                const float sl2 = a.q_prescaled ? 1.f : attn_q_scale(DH);
                hipLaunchKernelGGL((attn_merge_kernel<T, DH>), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s,
                                   a.kvpart, S, a.B, a.heads, a.N, sl2, (T *)a.out);
            } else {
                AttnArgs a1 = a;
                a1.kvsplit = 1;
                hipLaunchKernelGGL((attn_kernel<T, DH>), grid, dim3(256), 0, s, a1, q_start, n_qtiles);
            }
        }
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_dh(const AttnArgs &a, hipStream_t s) {
    return a.dh == 32 ? launch_t<T, 32>(a, s) : launch_t<T, 64>(a, s);
}

}  // namespace

hipError_t launch_attention(int act_dt, const AttnArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.N <= 0 || a.heads <= 0 || a.heads > 65535 || a.B > 65535 || a.N / QT >= 65535)
        return hipErrorInvalidValue;
    if (a.dh != 32 && a.dh != 64) return hipErrorInvalidValue;
    const int DH = a.dh;
    if (a.npad < cdiv(a.N, 64) * 64 || a.npad % 64) return hipErrorInvalidValue;
    // the 16-bit kernel addresses one item's rows with 32-bit byte offsets
    if ((int64_t)(a.N + 64) * a.ld_qk * 2 >= (1ll << 31) || (int64_t)DH * a.npad * 2 >= (1ll << 31))
        return hipErrorInvalidValue;
    if (a.ld_qk < 2 * (int64_t)a.heads * DH || a.ld_qk % 8) return hipErrorInvalidValue;
    if (((uintptr_t)a.qk | (uintptr_t)a.vt) % 16) return hipErrorInvalidValue;
    if (a.block_causal && (a.per_slot <= 0 || (a.N - a.has_cls) % a.per_slot)) return hipErrorInvalidValue;
    switch (act_dt) {
        case DT_F32: return launch_dh<float>(a, s);
        case DT_BF16: return launch_dh<bf16_t>(a, s);
        case DT_F16: return launch_dh<f16_t>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_xattn(int act_dt, const void *q, const void *k, const void *v, int64_t ldkv, int B, int N,
                        int heads, int dh, void *out, hipStream_t s) {
    if (B <= 0 || B > 65535 || N <= 0 || N > XATTN_MAX_N || heads <= 0 || heads > 65535 || (dh != 32 && dh != 64))
        return hipErrorInvalidValue;
    const int es = act_dt == DT_F32 ? 4 : 2;
    if (ldkv < (int64_t)heads * dh || (ldkv * es) % 16 || ((uintptr_t)k | (uintptr_t)v) % 16) return hipErrorInvalidValue;
    const dim3 grid(heads, B);
#define XA(T, DH_) hipLaunchKernelGGL((xattn_kernel<T, DH_>), grid, dim3(256), 0, s, (const T *)q, (const T *)k, \
                                      (const T *)v, ldkv, N, heads, (T *)out)
    switch (act_dt) {
        case DT_F32: if (dh == 32) XA(float, 32); else XA(float, 64); break;
        case DT_BF16: if (dh == 32) XA(bf16_t, 32); else XA(bf16_t, 64); break;
        case DT_F16: if (dh == 32) XA(f16_t, 32); else XA(f16_t, 64); break;
        default: return hipErrorInvalidValue;
    }
#undef XA
    return hipGetLastError();
}

hipError_t launch_transpose_v(int act_dt, const void *qkv, int B, int N, int D, void *vt,
                              int64_t npad, hipStream_t s) {
    if (B <= 0 || N <= 0 || D <= 0 || D % 64 || npad < cdiv(N, 16) * 16) return hipErrorInvalidValue;
    const dim3 grid((unsigned)cdiv(N, 64), D / 64, B);
    switch (act_dt) {
        case DT_F32:
            hipLaunchKernelGGL(transpose_v_kernel<float>, grid, dim3(256), 0, s, (const float *)qkv, N, D, (float *)vt, npad);
            break;
        case DT_BF16:
            hipLaunchKernelGGL(transpose_v_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t *)qkv, N, D, (bf16_t *)vt, npad);
            break;
        case DT_F16:
            hipLaunchKernelGGL(transpose_v_kernel<f16_t>, grid, dim3(256), 0, s, (const f16_t *)qkv, N, D, (f16_t *)vt, npad);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace jepa
