// The C ABI of include/jepa_mi355x.h: weight upload, workspace, the launch
// sequence of one encoder forward, pooling, timing and the host quantizer.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/jepa_mi355x.h"
#include "../../include/jepa_mi355x_ops.h"
#include "host.hpp"
#include "kernels.hpp"

using namespace jepa;

namespace {
thread_local std::string g_err;
}  // namespace

// the message jepa_last_error returns (host.hpp)
jepa_status jepa::fail(jepa_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

namespace {

#define HIP_TRY(expr)                                                                      \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess)                                                              \
            return fail(JEPA_E_HIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                        __LINE__);                                                         \
    } while (0)

// ---- host-side number formats ---------------------------------------------
uint16_t f32_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
float bf16_bits_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}
float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

// f32 -> IEEE half, round to nearest even.  Normal results round the
// mantissa with the usual add-half-minus-one-plus-odd-bit trick; results
// below the smallest normal half are produced by one f32 addition of a
// magic constant whose ulp is the half subnormal step, so the FPU's own
// round-to-nearest-even does the rounding.
uint16_t f32_to_f16_bits(float f) {
    uint32_t x = f32_bits(f);
    const uint32_t sign = x & 0x80000000u;
    x ^= sign;
    uint16_t o;
    if (x >= (143u << 23)) {                       // >= 65536, inf or nan
        o = x > (255u << 23) ? 0x7e00 : 0x7c00;
    } else if (x < (113u << 23)) {                 // below 2^-14
        const uint32_t magic = 126u << 23;         // 0.5: ulp 2^-24
        o = (uint16_t)(f32_bits(bits_f32(x) + bits_f32(magic)) - magic);
    } else {
        const uint32_t odd = (x >> 13) & 1u;
        x += 0xc8000fffu + odd;                    // rebias exponent (-112 << 23) and round
        o = (uint16_t)(x >> 13);
    }
    return (uint16_t)(o | (sign >> 16));
}
float f16_bits_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0) {
        const float v = (float)m * 5.9604644775390625e-08f;   // m * 2^-24, exact
        return sign ? -v : v;
    }
    if (e == 31) return bits_f32(sign | 0x7f800000u | (m << 13));
    return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

size_t storage_bytes(int dt, int64_t n) {
    switch (dt) {
        case JEPA_F32: return (size_t)n * 4;
        case JEPA_F16:
        case JEPA_BF16: return (size_t)n * 2;
        case JEPA_Q8_0: return (size_t)(n / 32) * 34;
        case JEPA_Q4_0: return (size_t)(n / 32) * 18;
        case JEPA_Q4_K: return (size_t)(n / 256) * 144;
        case JEPA_Q6_K: return (size_t)(n / 256) * 210;
    }
    return 0;
}

bool is_block_dt(int dt) { return dt == JEPA_Q8_0 || dt == JEPA_Q4_0 || dt == JEPA_Q4_K || dt == JEPA_Q6_K; }
bool is_kquant_dt(int dt) { return dt == JEPA_Q4_K || dt == JEPA_Q6_K; }

float stored_to_f32(int dt, const void *data, int64_t i) {
    switch (dt) {
        case JEPA_F32: return ((const float *)data)[i];
        case JEPA_F16: return f16_bits_to_f32(((const uint16_t *)data)[i]);
        case JEPA_BF16: return bf16_bits_to_f32(((const uint16_t *)data)[i]);
    }
    return NAN;
}

const char *kClassNames[] = {"patchify", "gemm_patch", "cls_rows", "layernorm", "gemm_qkv",
                             "transpose_v", "attention", "gemm_out", "gemm_fc1", "gemm_fc2",
                             "final_ln", "pool", "expand_weights", "head", "quant_act"};
enum KClass { K_PATCHIFY, K_GEMM_PATCH, K_CLS_ROWS, K_LN, K_GEMM_QKV, K_TRANSPOSE_V, K_ATTN,
              K_GEMM_OUT, K_GEMM_FC1, K_GEMM_FC2, K_FINAL_LN, K_POOL, K_EXPAND, K_HEAD, K_QUANT_ACT, K_COUNT };

struct DevTensor {
    void *ptr = nullptr;        // device data
    uint16_t *scale = nullptr;  // block formats: f16 scales (K-quants: per super-block)
    const uint8_t *sub = nullptr;   // K-quants: the sub-block scale bytes
    int dev_dt = 0;             // device dtype
    int64_t ne0 = 0, ne1 = 0;
};

struct Layer {
    DevTensor qkv, out, up, down;
    DevTensor xqkv, xout, xup, xdown;   // block-format ones expanded to the act dtype (when in use)
    float *ln1g, *ln1b, *ln2g, *ln2b, *bqkv, *bout, *bup, *bdown;
};

// The attentive-pool classifier head's cross-attention block and classifier
// (its self-attention blocks are Layers).  The classifier's rows are padded
// with zero rows to Cpad, a multiple of 64.
struct Head {
    int C = 0, Cpad = 0;
    float *q0 = nullptr, *ln1g = nullptr, *ln1b = nullptr, *ln2g = nullptr, *ln2b = nullptr;
    DevTensor wq, wk, wv, wo, wup, wdown, wc;
    DevTensor xwq, xwk, xwv, xwo, xwup, xwdown;   // block-format ones expanded (when in use)
    float *bq = nullptr, *bk = nullptr, *bv = nullptr, *bo = nullptr, *bup = nullptr, *bdown = nullptr,
          *bc = nullptr;
};

struct ProfRec {
    int cls;
    hipEvent_t a, b;
};

// Device buffers of one encode (rows of a batch); see ws_layout.
struct Ws {
    uint8_t *frames = nullptr;   // host frames staged to the device
    void *patch = nullptr, *hn = nullptr, *qkv = nullptr, *vt = nullptr, *o = nullptr, *u = nullptr;
    float *x = nullptr, *y = nullptr, *pool = nullptr;
    // classifier head: x rows f32, LN / cast output, query, attention out,
    // MLP hidden (act dtype), padded scores f32
    float *hx = nullptr, *hl = nullptr;
    void *hh = nullptr, *hq = nullptr, *ho = nullptr, *hu = nullptr;
    float *kpart = nullptr, *kvpart = nullptr;   // f32 models: split partials
    // int8 path: a product's input quantised per 32-block, codes [rows,
    // max(D, F)] and f32 scales [rows, max(D, F) / 32]
    int8_t *qa = nullptr;
    float *qas = nullptr;
};

}  // namespace

struct jepa_ctx {
    jepa_dims d;
    int D, H, F, L, P, Kp, Np, N, per_slot, act, es;
    int64_t npad;               // V^T row length: N rounded up to 64
    void *arena = nullptr;
    size_t arena_bytes = 0, model_bytes = 0;
    DevTensor wpe;
    float *bpe = nullptr, *cls = nullptr, *pos = nullptr, *normg = nullptr, *normb = nullptr;
    float *rope = nullptr;      // 3-D rotary table [N, 32] (cos, sin), or null
    // pixel normalisation as one f32 FMA per value, u * pix_scale[c] +
    // pix_shift[c] (1/(255 std_c) and -mean_c/std_c, rounded once from double)
    float pix_scale[3] = {}, pix_shift[3] = {};
    // block-format matrices expanded to the act dtype for large batches (and
    // always when a K-quant matrix is present)
    bool has_q = false, has_k = false;
    void *xbuf = nullptr;       // expansion jobs, then the expanded matrices
    size_t xbuf_bytes = 0;
    const ExpandJob *xjobs = nullptr;
    int n_xjobs = 0;
    int64_t x_nblk = 0;
    // the copy depends on the weights alone, which never change after
    // create: it is written by the first encode that uses it (x_written,
    // recorded by x_ev on that encode's stream) and read by every later one
    bool x_written = false;
    hipEvent_t x_ev = nullptr;
    std::vector<Layer> layers, head_layers;
    Head head;
    std::map<std::string, DevTensor> by_name;
    // workspace
    void *ws = nullptr;
    size_t ws_bytes = 0;
    int ws_batch = 0;
    // host frames are staged through this pinned buffer; h_ev marks the end
    // of the last copy out of it
    uint8_t *h_frames = nullptr;
    size_t h_frames_bytes = 0;
    hipEvent_t h_ev = nullptr;
    bool h_pending = false;
    Ws w;                       // the workspace's buffers
    bool last_expand = false;   // the last encode used the expanded matrices
    bool int8_mm = false;       // jepa_set_int8_matmul: q8_0 / q4_0 products on int8 MFMA
    // last encode
    const float *last_tokens = nullptr;
    int last_batch = 0;
    bool have_events = false, encoded = false;
    hipEvent_t ev0, ev1;
    // batch parts run on the caller's stream and up to MAX_PARTS-1 of these
    // (forked from and joined back onto the caller's stream); four streams in
    // all match the four hardware queues HIP gives a process by default
    static constexpr int MAX_PARTS = 4;
    int parts_set = 0;          // jepa_set_batch_parts (0 = default)
    hipStream_t aux[MAX_PARTS - 1] = {};
    hipEvent_t fork_ev = nullptr, join_ev[MAX_PARTS - 1] = {};
    // profiling
    uint32_t prof = 0;          // class bitmask
    std::vector<ProfRec> pending;
    std::vector<hipEvent_t> event_pool;
    int64_t stat_launches[K_COUNT] = {};
    double stat_ms[K_COUNT] = {};
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t frames, patch, x, hn, qkv, vt, o, u, y, pool, hx, hh, hq, ho, hu, hl, kpart, kvpart, qa, qas, total;
};

// with_frames: a region for host frames staged to the device
WsLayout ws_layout(const jepa_ctx *c, int B, bool with_frames = true) {
    WsLayout w;
    const size_t M = (size_t)B * c->N;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    w.frames = take(with_frames ? (size_t)B * c->d.frames * c->d.img_h * c->d.img_w * 3 : 0);
    w.patch = take((size_t)B * c->Np * c->Kp * c->es);
    w.x = take(M * c->D * 4);
    w.hn = take(M * c->D * c->es);
    w.qkv = take(M * 3 * c->D * c->es);
    w.vt = take((size_t)B * c->D * c->npad * c->es);
    w.o = take(M * c->D * c->es);
    w.u = take(M * c->F * c->es);
    w.y = take(M * c->D * 4);
    w.pool = take((size_t)B * POOL_CHUNKS * c->D * 4);
    // the classifier head's rows (one per item)
    const size_t hb = c->head.C > 0 ? (size_t)B : 0;
    w.hx = take(hb * c->D * 4);
    w.hh = take(hb * c->D * c->es);
    w.hq = take(hb * c->D * c->es);
    w.ho = take(hb * c->D * c->es);
    w.hu = take(hb * c->F * c->es);
    w.hl = take(hb * c->head.Cpad * 4);
    // f32 models (small ones) split long residual GEMMs and attention over
    // few workgroups; their partial results
    const bool f32 = c->act == JEPA_F32;
    w.kpart = take(f32 ? (size_t)KSPLIT_MAX * M * c->D * 4 : 0);
    w.kvpart = take(f32 ? (size_t)KVSPLIT_MAX * M * c->H * (c->D / c->H + 2) * 4 : 0);
    const size_t kf = (size_t)std::max(c->D, c->F);
    w.qa = take(c->int8_mm ? M * kf : 0);
    w.qas = take(c->int8_mm ? M * (kf / 32) * 4 : 0);
    w.total = off;
    return w;
}

// Large batches run the block-format layers as dense GEMMs on an act-dtype
// copy of the block matrices, expanded by the first encode that needs it (a
// bandwidth-bound pass: 1 + 1/16 bytes read and 2 written per weight for
// q8_0) and kept, like the weights, until the context is freed.  Above ~1024
// rows per batch part the GEMMs take the 256-row MFMA tiles, whose operands
// flow straight from memory into LDS; a dequantising load would put the
// conversion on the VALU inside the K loop, and an int8 MFMA path with
// per-block rescaling is VALU-bound on this chip.  Small batches keep the
// dequantising 128 x 128 tile for q8_0 / q4_0; the K-quants (whose 256-weight
// super-blocks straddle that tile's 64-wide K steps) are always expanded.
// JEPA_Q_EXPAND = 0 / 1 forces either for models without K-quants.
// Every (block matrix, its expanded copy) pair: the encoder's blocks, the
// classifier head's blocks and its cross-attention matrices.
std::vector<std::pair<DevTensor *, DevTensor *>> expand_pairs(jepa_ctx *c) {
    std::vector<std::pair<DevTensor *, DevTensor *>> v;
    auto add = [&](DevTensor &t, DevTensor &x) { v.emplace_back(&t, &x); };
    for (auto *Ls : {&c->layers, &c->head_layers})
        for (Layer &L : *Ls) {
            add(L.qkv, L.xqkv); add(L.out, L.xout); add(L.up, L.xup); add(L.down, L.xdown);
        }
    if (c->head.C > 0) {
        Head &h = c->head;
        add(h.wq, h.xwq); add(h.wk, h.xwk); add(h.wv, h.xwv); add(h.wo, h.xwo);
        add(h.wup, h.xwup); add(h.wdown, h.xwdown);
    }
    return v;
}

size_t expand_bytes(const jepa_ctx *c) {
    size_t n = 0, jobs = 0;
    for (auto &pr : expand_pairs(const_cast<jepa_ctx *>(c)))
        if (is_block_dt(pr.first->dev_dt)) {
            n += align256((size_t)pr.first->ne0 * pr.first->ne1 * c->es);
            ++jobs;
        }
    return jobs ? align256(jobs * sizeof(ExpandJob)) + n : 0;
}

bool use_expand(const jepa_ctx *c, int batch, int parts) {
    if (!c->has_q) return false;
    if (c->has_k) return true;
    if (c->int8_mm) return false;   // the int8 path reads the blocks themselves
    if (const char *e = getenv("JEPA_Q_EXPAND")) {
        if (!strcmp(e, "0")) return false;
        if (!strcmp(e, "1")) return true;
    }
    return (int64_t)((batch + parts - 1) / parts) * c->N >= 1024;
}

jepa_status ensure_expanded(jepa_ctx *c) {
    if (c->xbuf) return JEPA_OK;
    const size_t bytes = expand_bytes(c);
    if (hipMalloc(&c->xbuf, bytes) != hipSuccess) {
        c->xbuf = nullptr;
        (void)hipGetLastError();
        return fail(JEPA_E_OOM, "hipMalloc of %zu bytes for the expanded block matrices failed", bytes);
    }
    const auto pairs = expand_pairs(c);
    size_t n_jobs = 0;
    for (auto &pr : pairs) n_jobs += is_block_dt(pr.first->dev_dt);
    unsigned char *base = (unsigned char *)c->xbuf;
    size_t off = align256(n_jobs * sizeof(ExpandJob));
    std::vector<ExpandJob> jobs;
    int64_t blk = 0;
    for (auto &pr : pairs) {
        const DevTensor &t = *pr.first;
        DevTensor &x = *pr.second;
        x = t;
        if (!is_block_dt(t.dev_dt)) continue;
        x.dev_dt = c->act;
        x.scale = nullptr;
        x.sub = nullptr;
        x.ptr = base + off;
        jobs.push_back(ExpandJob{t.ptr, t.scale, t.sub, x.ptr, blk, t.dev_dt});
        blk += t.ne0 * t.ne1 / 32;
        off += align256((size_t)t.ne0 * t.ne1 * c->es);
    }
    if (hipMemcpy(c->xbuf, jobs.data(), jobs.size() * sizeof(ExpandJob), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(c->xbuf);
        c->xbuf = nullptr;
        return fail(JEPA_E_HIP, "upload of the expansion jobs failed");
    }
    c->xbuf_bytes = bytes;
    c->xjobs = (const ExpandJob *)c->xbuf;
    c->n_xjobs = (int)jobs.size();
    c->x_nblk = blk;
    return JEPA_OK;
}

// The buffers of layout w at device address base.
Ws ws_pointers(const jepa_ctx *c, const WsLayout &w, unsigned char *base) {
    Ws p;
    p.frames = base + w.frames;
    p.patch = base + w.patch;
    p.x = (float *)(base + w.x);
    p.hn = base + w.hn;
    p.qkv = base + w.qkv;
    p.vt = base + w.vt;
    p.o = base + w.o;
    p.u = base + w.u;
    p.y = (float *)(base + w.y);
    p.pool = (float *)(base + w.pool);
    p.hx = (float *)(base + w.hx);
    p.hh = base + w.hh;
    p.hq = base + w.hq;
    p.ho = base + w.ho;
    p.hu = base + w.hu;
    p.hl = (float *)(base + w.hl);
    p.kpart = c->act == JEPA_F32 ? (float *)(base + w.kpart) : nullptr;
    p.kvpart = c->act == JEPA_F32 ? (float *)(base + w.kvpart) : nullptr;
    p.qa = c->int8_mm ? (int8_t *)(base + w.qa) : nullptr;
    p.qas = c->int8_mm ? (float *)(base + w.qas) : nullptr;
    return p;
}

// Forget every pointer into the workspace (before it is freed).
void clear_workspace(jepa_ctx *c) {
    c->w = Ws{};
    c->ws_bytes = 0;
    c->ws_batch = 0;
}

// Free the workspace once the device is idle; nothing may keep pointing into
// it afterwards (the next encode allocates it again).
jepa_status release_workspace(jepa_ctx *c) {
    if (!c->ws) return JEPA_OK;
    c->encoded = false;
    c->last_tokens = nullptr;
    c->last_batch = 0;
    HIP_TRY(hipDeviceSynchronize());
    clear_workspace(c);
    HIP_TRY(hipFree(c->ws));
    c->ws = nullptr;
    return JEPA_OK;
}

jepa_status ensure_workspace(jepa_ctx *c, int B) {
    if (B <= c->ws_batch) return JEPA_OK;
    WsLayout w = ws_layout(c, B);
    const char *cap = getenv("JEPA_MAX_WORKSPACE");
    if (cap && (double)w.total > atof(cap))
        return fail(JEPA_E_OOM, "workspace of %zu bytes for batch %d exceeds JEPA_MAX_WORKSPACE=%s",
                    w.total, B, cap);
    if (const jepa_status st = release_workspace(c)) return st;
    if (hipMalloc(&c->ws, w.total) != hipSuccess) {
        c->ws = nullptr;
        (void)hipGetLastError();
        return fail(JEPA_E_OOM, "hipMalloc of %zu workspace bytes failed", w.total);
    }
    c->w = ws_pointers(c, w, (unsigned char *)c->ws);
    // columns N..npad-1 of V^T are read (and multiplied by zero weights) by
    // the last key tile of each head: keep them finite
    HIP_TRY(hipMemset(c->w.vt, 0, (size_t)B * c->D * c->npad * c->es));
    c->ws_bytes = w.total;
    c->ws_batch = B;
    return JEPA_OK;
}

hipEvent_t get_event(jepa_ctx *c) {
    if (!c->event_pool.empty()) {
        hipEvent_t e = c->event_pool.back();
        c->event_pool.pop_back();
        return e;
    }
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launch wrapper: brackets the launch with events when profiling is on.
template <typename F>
jepa_status launch(jepa_ctx *c, int cls, hipStream_t s, F &&fn) {
    ProfRec r{cls, nullptr, nullptr};
    const bool on = (c->prof >> cls) & 1u;
    if (on) {
        r.a = get_event(c);
        r.b = get_event(c);
        if (r.a) HIP_TRY(hipEventRecord(r.a, s));
    }
    hipError_t e = fn();
    if (e != hipSuccess) return fail(JEPA_E_HIP, "%s launch failed: %s", kClassNames[cls], hipGetErrorString(e));
    if (on && r.a && r.b) {
        HIP_TRY(hipEventRecord(r.b, s));
        c->pending.push_back(r);
    }
    return JEPA_OK;
}

#define TRY(expr)                       \
    do {                                \
        jepa_status st_ = (expr);       \
        if (st_ != JEPA_OK) return st_; \
    } while (0)

jepa_status check_dims(const jepa_dims *d) {
    if (d->dim <= 0 || d->depth <= 0 || d->heads <= 0 || d->mlp_dim <= 0 || d->patch <= 0 ||
        d->tubelet <= 0 || d->img_h <= 0 || d->img_w <= 0 || d->frames <= 0)
        return fail(JEPA_E_SHAPE, "dims: every size must be positive");
    if (d->dim % d->heads || (d->dim / d->heads != 64 && d->dim / d->heads != 32))
        return fail(JEPA_E_UNSUPPORTED, "dims: head_dim = dim/heads must be 32 or 64 (dim %d, heads %d)", d->dim, d->heads);
    if (d->dim % 64 || d->mlp_dim % 64)
        return fail(JEPA_E_UNSUPPORTED, "dims: dim and mlp_dim must be multiples of 64");
    const int e = d->dim / 64;
    if (!(e == 2 || e == 3 || e == 4 || e == 6 || e == 8 || e == 12 || e == 16 || e == 20 || e == 24 || e == 32))
        return fail(JEPA_E_UNSUPPORTED, "dims: dim %d not among the LayerNorm widths built", d->dim);
    if (d->img_h % d->patch || d->img_w % d->patch)
        return fail(JEPA_E_SHAPE, "dims: img_h, img_w must be multiples of patch");
    if (d->frames % d->tubelet) return fail(JEPA_E_SHAPE, "dims: frames %% tubelet != 0");
    if (d->has_cls != 0 && d->has_cls != 1) return fail(JEPA_E_INVALID_ARG, "dims: has_cls must be 0 or 1");
    if (d->rope != 0 && d->rope != 1) return fail(JEPA_E_INVALID_ARG, "dims: rope must be 0 or 1");
    if (d->head_blocks < 0 || d->head_classes < 0 || d->head_blocks > 64 || d->head_classes > (1 << 20))
        return fail(JEPA_E_INVALID_ARG, "dims: head_blocks %d / head_classes %d out of range", d->head_blocks,
                    d->head_classes);
    if (d->mask != JEPA_MASK_BIDIR && d->mask != JEPA_MASK_BLOCK_CAUSAL)
        return fail(JEPA_E_INVALID_ARG, "dims: unknown mask %d", d->mask);
    if (d->act_dtype != JEPA_F32 && d->act_dtype != JEPA_F16 && d->act_dtype != JEPA_BF16)
        return fail(JEPA_E_DTYPE, "dims: act_dtype must be F32, F16 or BF16");
    if (!(d->ln_eps > 0.f)) return fail(JEPA_E_INVALID_ARG, "dims: ln_eps must be > 0");
    for (int c = 0; c < 3; ++c)
        if (!(d->std[c] != 0.f)) return fail(JEPA_E_INVALID_ARG, "dims: std[%d] is 0", c);
    return JEPA_OK;
}

// 3-D rotary position (V-JEPA 2 card, opening paragraph; RoFormer's pairwise
// rotation): [N, dh/2] (cos, sin) pairs, three segments of ds = 2*floor(dh/6)
// dims (20 of 64, 10 of 32) for the temporal slot, patch row and patch
// column, pair i of a segment at frequency 10000^(-2i/ds); the pairs past
// the three segments and every pair of a CLS token have angle 0.
void rope_table(const jepa_dims &d, float *out) {
    const int dh = d.dim / d.heads, np = dh / 2, ds = 2 * (dh / 6);
    const int Hp = d.img_h / d.patch, Wp = d.img_w / d.patch;
    const int Np = d.frames / d.tubelet * Hp * Wp, N = Np + d.has_cls;
    for (int n = 0; n < N; ++n) {
        float *row = out + (size_t)n * dh;
        for (int p = 0; p < np; ++p) { row[2 * p] = 1.f; row[2 * p + 1] = 0.f; }
        if (d.has_cls && n == 0) continue;
        const int pn = n - d.has_cls;
        const int pos[3] = {pn / (Hp * Wp), pn / Wp % Hp, pn % Wp};
        for (int a = 0; a < 3; ++a)
            for (int i = 0; i < ds / 2; ++i) {
                const double ang = pos[a] * pow(10000.0, -2.0 * i / ds);
                row[2 * (a * ds / 2 + i)] = (float)cos(ang);
                row[2 * (a * ds / 2 + i) + 1] = (float)sin(ang);
            }
    }
}

// [blocks](f16 scale, payload) -> payloads then scales
void pack_blocks(int dt, const unsigned char *src, int64_t nb, unsigned char *codes, uint16_t *scales) {
    const int bb = dt == JEPA_Q8_0 ? 34 : 18, pl = bb - 2;
    for (int64_t ib = 0; ib < nb; ++ib) {
        memcpy(codes + ib * pl, src + ib * bb + 2, pl);
        memcpy(scales + ib, src + ib * bb, 2);
    }
}

// K-quant super-blocks as stored -> codes, f16 scales, sub-block scale bytes
// (the device layout; no value changes).  q4_K (144 bytes): d, dmin, 12
// scale bytes, 128 code bytes.  q6_K (210 bytes): 128 low-bit and 64
// high-bit code bytes, 16 int8 scales, d.
void pack_superblocks(int dt, const unsigned char *src, int64_t nsb, unsigned char *codes, uint16_t *scales,
                      unsigned char *sub) {
    for (int64_t i = 0; i < nsb; ++i) {
        if (dt == JEPA_Q4_K) {
            const unsigned char *b = src + i * 144;
            memcpy(scales + 2 * i, b, 4);
            memcpy(sub + i * 12, b + 4, 12);
            memcpy(codes + i * 128, b + 16, 128);
        } else {
            const unsigned char *b = src + i * 210;
            memcpy(codes + i * 192, b, 192);
            memcpy(sub + i * 16, b + 192, 16);
            memcpy(scales + i, b + 208, 2);
        }
    }
}

struct Expect {
    int64_t ne0, ne1;
    bool matrix;      // may be re-typed to a block format
    bool present = false;
    const jepa_tensor *t = nullptr;
};

}  // namespace

// ---------------------------------------------------------------------------
// The no-allocation encode's buffers: one static device array, one copy per
// device.  Host code never uses the array's name as an address: each
// device's copy is looked up once, with that device current, and kept here.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[JEPA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// The current device's address of `scratch` (looked up on first use).
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

extern "C" {

const char *jepa_last_error(void) { return g_err.c_str(); }

jepa_status jepa_quantize(int dtype, const float *src, int64_t rows, int64_t cols, uint8_t *dst) {
#pragma clang fp contract(off)
    if (!src || !dst || rows <= 0 || cols <= 0) return fail(JEPA_E_INVALID_ARG, "quantize: bad arguments");
    if (cols % 32) return fail(JEPA_E_SHAPE, "quantize: cols %lld not a multiple of 32", (long long)cols);
    if (dtype != JEPA_Q8_0 && dtype != JEPA_Q4_0) return fail(JEPA_E_DTYPE, "quantize: dtype must be Q8_0 or Q4_0");
    const int64_t nb = rows * (cols / 32);
    for (int64_t ib = 0; ib < nb; ++ib) {
        const float *x = src + ib * 32;
        float d;
        uint8_t *o;
        if (dtype == JEPA_Q8_0) {
            float amax = 0.f;
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
            d = amax / 127.f;
            const float id = d != 0.f ? 1.f / d : 0.f;
            o = dst + ib * 34;
            for (int j = 0; j < 32; ++j) ((int8_t *)o)[2 + j] = (int8_t)roundf(x[j] * id);
        } else {
            float amax = 0.f, m = 0.f;
            for (int j = 0; j < 32; ++j)
                if (amax < fabsf(x[j])) { amax = fabsf(x[j]); m = x[j]; }
            d = m / -8.f;
            const float id = d != 0.f ? 1.f / d : 0.f;
            o = dst + ib * 18;
            for (int j = 0; j < 16; ++j) {
                int q0 = (int)(x[j] * id + 8.5f), q1 = (int)(x[j + 16] * id + 8.5f);
                q0 = q0 < 15 ? q0 : 15;
                q1 = q1 < 15 ? q1 : 15;
                o[2 + j] = (uint8_t)(q0 | (q1 << 4));
            }
        }
        const uint16_t h = f32_to_f16_bits(d);
        memcpy(o, &h, 2);
    }
    return JEPA_OK;
}

jepa_status jepa_create(const jepa_dims *dims, const jepa_tensor *tensors, int n_tensors, jepa_ctx **out) {
    if (!dims || !out || (!tensors && n_tensors > 0) || n_tensors < 0)
        return fail(JEPA_E_INVALID_ARG, "create: null argument");
    *out = nullptr;
    TRY(check_dims(dims));
    const jepa_dims &d = *dims;
    const int D = d.dim, F = d.mlp_dim;
    const int Tt = d.frames / d.tubelet, Hp = d.img_h / d.patch, Wp = d.img_w / d.patch;
    const int Np = Tt * Hp * Wp, N = Np + d.has_cls, P = d.tubelet * d.patch * d.patch * 3;

    // expected schema
    std::map<std::string, Expect> want;
    want["enc.patch_embed.weight"] = {P, D, false};
    want["enc.patch_embed.bias"] = {D, 1, false};
    if (d.has_cls) want["enc.cls_token"] = {D, 1, false};
    if (!d.rope) want["enc.pos_embed"] = {D, N, false};
    want["enc.norm.weight"] = {D, 1, false};
    want["enc.norm.bias"] = {D, 1, false};
    auto want_block = [&](const std::string &p) {
        want[p + "ln1.weight"] = {D, 1, false};
        want[p + "ln1.bias"] = {D, 1, false};
        want[p + "ln2.weight"] = {D, 1, false};
        want[p + "ln2.bias"] = {D, 1, false};
        want[p + "attn_qkv.weight"] = {D, 3 * D, true};
        want[p + "attn_qkv.bias"] = {3 * D, 1, false};
        want[p + "attn_out.weight"] = {D, D, true};
        want[p + "attn_out.bias"] = {D, 1, false};
        want[p + "ffn_up.weight"] = {D, F, true};
        want[p + "ffn_up.bias"] = {F, 1, false};
        want[p + "ffn_down.weight"] = {F, D, true};
        want[p + "ffn_down.bias"] = {D, 1, false};
    };
    for (int i = 0; i < d.depth; ++i) want_block("enc.blk." + std::to_string(i) + ".");
    // the attentive-pool classifier head: its blocks, the cross-attention
    // query block (query token, ln1 on the tokens, q / k / v / out, ln2, MLP)
    // and the classifier
    const int C = d.head_classes, Cpad = (C + 63) / 64 * 64;
    if (C > 0) {
        for (int i = 0; i < d.head_blocks; ++i) want_block("head.blk." + std::to_string(i) + ".");
        const std::string p = "head.xattn.";
        want["head.query_token"] = {D, 1, false};
        for (const char *n : {"ln1", "ln2"}) {
            want[p + n + ".weight"] = {D, 1, false};
            want[p + n + ".bias"] = {D, 1, false};
        }
        for (const char *n : {"attn_q", "attn_k", "attn_v", "attn_out"}) {
            want[p + n + ".weight"] = {D, D, true};
            want[p + n + ".bias"] = {D, 1, false};
        }
        want[p + "ffn_up.weight"] = {D, F, true};
        want[p + "ffn_up.bias"] = {F, 1, false};
        want[p + "ffn_down.weight"] = {F, D, true};
        want[p + "ffn_down.bias"] = {D, 1, false};
        want["head.classifier.weight"] = {D, C, false};
        want["head.classifier.bias"] = {C, 1, false};
    }
    size_t model_bytes = 0;
    for (int i = 0; i < n_tensors; ++i) {
        const jepa_tensor &t = tensors[i];
        if (!t.name) return fail(JEPA_E_INVALID_ARG, "create: tensor %d has no name", i);
        auto it = want.find(t.name);
        if (it == want.end()) return fail(JEPA_E_INVALID_ARG, "create: unknown tensor '%s'", t.name);
        Expect &e = it->second;
        if (e.present) return fail(JEPA_E_INVALID_ARG, "create: tensor '%s' given twice", t.name);
        if (t.ne0 != e.ne0 || t.ne1 != e.ne1)
            return fail(JEPA_E_SHAPE, "create: '%s' is [%lld, %lld], expected [%lld, %lld]", t.name,
                        (long long)t.ne0, (long long)t.ne1, (long long)e.ne0, (long long)e.ne1);
        if (t.dtype < JEPA_F32 || t.dtype > JEPA_Q6_K)
            return fail(JEPA_E_DTYPE, "create: '%s' has unknown dtype %d", t.name, t.dtype);
        if (is_block_dt(t.dtype) && !e.matrix)
            return fail(JEPA_E_DTYPE, "create: '%s' must keep a dense dtype (only the block matrices may be re-typed)", t.name);
        if (is_block_dt(t.dtype) && (t.ne0 % 64))
            return fail(JEPA_E_SHAPE, "create: '%s' row length %lld not a multiple of 64 for block formats", t.name, (long long)t.ne0);
        if (is_kquant_dt(t.dtype) && (t.ne0 % 256))
            return fail(JEPA_E_SHAPE, "create: '%s' row length %lld not a multiple of 256 for a K-quant (such rows "
                        "take q4_0 / q8_0 instead)", t.name, (long long)t.ne0);
        if (is_block_dt(t.dtype) && d.act_dtype == JEPA_F32)
            return fail(JEPA_E_UNSUPPORTED, "create: block-format '%s' needs act_dtype F16 or BF16", t.name);
        const size_t nb = storage_bytes(t.dtype, t.ne0 * t.ne1);
        if (t.nbytes != nb)
            return fail(JEPA_E_SHAPE, "create: '%s' has %zu bytes, its dtype and shape need %zu", t.name, t.nbytes, nb);
        if (!t.data) return fail(JEPA_E_INVALID_ARG, "create: '%s' has no data", t.name);
        e.present = true;
        e.t = &t;
        model_bytes += nb;
    }
    for (auto &kv : want)
        if (!kv.second.present) return fail(JEPA_E_MISSING_TENSOR, "create: tensor '%s' is missing", kv.first.c_str());

    jepa_ctx *c = new jepa_ctx();
    c->d = d;
    c->D = D; c->H = d.heads; c->F = F; c->L = d.depth; c->P = P;
    c->act = d.act_dtype;
    c->es = d.act_dtype == JEPA_F32 ? 4 : 2;
    const int bk = 128 / c->es;
    c->Kp = (P + bk - 1) / bk * bk;
    c->Np = Np; c->N = N; c->per_slot = Hp * Wp;
    c->npad = (N + 63) / 64 * 64;
    c->model_bytes = model_bytes;
    for (int i = 0; i < 3; ++i) {
        c->pix_scale[i] = (float)(1.0 / (255.0 * (double)d.std[i]));
        c->pix_shift[i] = (float)(-(double)d.mean[i] / (double)d.std[i]);
    }

    // device layout of every tensor: block matrices keep their format (codes
    // then scales); other matrices take the act dtype; vectors become f32.
    struct Plan { std::string name; const jepa_tensor *t; int dev_dt; size_t off, scale_off, sub_off, bytes; };
    std::vector<Plan> plan;
    size_t off = 0;
    for (auto &kv : want) {
        const jepa_tensor *t = kv.second.t;
        Plan p{kv.first, t, 0, 0, 0, 0, 0};
        // vectors and the pos table are consumed in f32 by the epilogues
        const bool vec = t->ne1 == 1 || kv.first == "enc.pos_embed";
        if (is_kquant_dt(t->dtype)) {
            // codes, then f16 scales, then the sub-block scale bytes
            const bool q4 = t->dtype == JEPA_Q4_K;
            const size_t nsb = (size_t)t->ne0 * t->ne1 / 256;
            p.dev_dt = t->dtype;
            p.off = off;
            p.bytes = nsb * (q4 ? 128 : 192);
            off += align256(p.bytes);
            p.scale_off = off;
            off += align256(nsb * (q4 ? 4 : 2));
            p.sub_off = off;
            off += align256(nsb * (q4 ? 12 : 16));
        } else if (t->dtype == JEPA_Q8_0 || t->dtype == JEPA_Q4_0) {
            p.dev_dt = t->dtype;
            p.off = off;
            const size_t codes = t->dtype == JEPA_Q8_0 ? (size_t)t->ne0 * t->ne1 : (size_t)t->ne0 * t->ne1 / 2;
            off += align256(codes);
            p.scale_off = off;
            off += align256((size_t)t->ne0 * t->ne1 / 32 * 2);
            p.bytes = codes;
        } else if (vec) {
            // (the classifier's bias padded with zeros to a multiple of 64)
            p.dev_dt = JEPA_F32;
            p.off = off;
            p.bytes = (size_t)(kv.first == "head.classifier.bias" ? Cpad : t->ne0) * t->ne1 * 4;
            off += align256(p.bytes);
        } else {
            // (the classifier's rows padded with zero rows to a multiple of 64)
            p.dev_dt = c->act;
            p.off = off;
            const int64_t rowlen = kv.first == "enc.patch_embed.weight" ? c->Kp : t->ne0;
            p.bytes = (size_t)rowlen * (kv.first == "head.classifier.weight" ? Cpad : t->ne1) * c->es;
            off += align256(p.bytes);
        }
        plan.push_back(p);
    }
    // the rotary table follows the weights
    const size_t rope_off = off;
    std::vector<float> rope_host;
    if (d.rope) {
        rope_host.resize((size_t)N * (D / d.heads));
        rope_table(d, rope_host.data());
        off += align256(rope_host.size() * 4);
    }
    if (hipMalloc(&c->arena, off) != hipSuccess) {
        (void)hipGetLastError();
        delete c;
        return fail(JEPA_E_OOM, "create: hipMalloc of %zu weight bytes failed", off);
    }
    c->arena_bytes = off;
    unsigned char *arena = (unsigned char *)c->arena;
    if (d.rope && hipMemcpy(arena + rope_off, rope_host.data(), rope_host.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
        jepa_free(c);
        return fail(JEPA_E_HIP, "create: upload of the rotary table failed");
    }

    std::vector<unsigned char> host;
    for (auto &p : plan) {
        const jepa_tensor *t = p.t;
        DevTensor dt;
        dt.dev_dt = p.dev_dt;
        dt.ne0 = t->ne0;
        dt.ne1 = t->ne1;
        dt.ptr = arena + p.off;
        const int64_t n = t->ne0 * t->ne1;
        if (is_kquant_dt(p.dev_dt)) {
            const bool q4 = p.dev_dt == JEPA_Q4_K;
            const int64_t nsb = n / 256;
            const size_t sbytes = nsb * (q4 ? 4 : 2), ubytes = nsb * (q4 ? 12 : 16);
            host.assign(p.bytes + sbytes + ubytes, 0);
            pack_superblocks(p.dev_dt, (const unsigned char *)t->data, nsb, host.data(),
                             (uint16_t *)(host.data() + p.bytes), host.data() + p.bytes + sbytes);
            dt.scale = (uint16_t *)(arena + p.scale_off);
            dt.sub = arena + p.sub_off;
            if (hipMemcpy(dt.ptr, host.data(), p.bytes, hipMemcpyHostToDevice) != hipSuccess ||
                hipMemcpy(dt.scale, host.data() + p.bytes, sbytes, hipMemcpyHostToDevice) != hipSuccess ||
                hipMemcpy((void *)dt.sub, host.data() + p.bytes + sbytes, ubytes, hipMemcpyHostToDevice) != hipSuccess) {
                jepa_free(c);
                return fail(JEPA_E_HIP, "create: upload of '%s' failed", p.name.c_str());
            }
        } else if (p.dev_dt == JEPA_Q8_0 || p.dev_dt == JEPA_Q4_0) {
            // repack [rows][blocks](scale, payload) into codes then scales
            const int64_t nb = n / 32;
            host.assign(p.bytes + nb * 2, 0);
            pack_blocks(p.dev_dt, (const unsigned char *)t->data, nb, host.data(),
                        (uint16_t *)(host.data() + p.bytes));
            dt.scale = (uint16_t *)(arena + p.scale_off);
            if (hipMemcpy(dt.ptr, host.data(), p.bytes, hipMemcpyHostToDevice) != hipSuccess ||
                hipMemcpy(dt.scale, host.data() + p.bytes, nb * 2, hipMemcpyHostToDevice) != hipSuccess) {
                jepa_free(c);
                return fail(JEPA_E_HIP, "create: upload of '%s' failed", p.name.c_str());
            }
        } else {
            host.assign(p.bytes, 0);
            const int64_t rowlen = p.name == "enc.patch_embed.weight" ? c->Kp : t->ne0;
            const int es = p.dev_dt == JEPA_F32 ? 4 : 2;
            if (p.dev_dt == t->dtype) {   // same format: copy rows (padded for patch-embed)
                for (int64_t r = 0; r < t->ne1; ++r)
                    memcpy(&host[r * rowlen * es], (const unsigned char *)t->data + r * t->ne0 * es, t->ne0 * es);
            } else {                      // widen exactly, or round to nearest even
                for (int64_t r = 0; r < t->ne1; ++r)
                    for (int64_t k = 0; k < t->ne0; ++k) {
                        const int64_t i = r * t->ne0 + k, o = r * rowlen + k;
                        const float v = stored_to_f32(t->dtype, t->data, i);
                        if (p.dev_dt == JEPA_F32) {
                            memcpy(&host[o * 4], &v, 4);
                        } else {
                            const uint16_t h = p.dev_dt == JEPA_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
                            memcpy(&host[o * 2], &h, 2);
                        }
                    }
            }
            if (hipMemcpy(dt.ptr, host.data(), p.bytes, hipMemcpyHostToDevice) != hipSuccess) {
                jepa_free(c);
                return fail(JEPA_E_HIP, "create: upload of '%s' failed", p.name.c_str());
            }
        }
        c->by_name[p.name] = dt;
    }
    auto vecp = [&](const std::string &n) { return (float *)c->by_name[n].ptr; };
    c->wpe = c->by_name["enc.patch_embed.weight"];
    c->bpe = vecp("enc.patch_embed.bias");
    c->cls = d.has_cls ? vecp("enc.cls_token") : nullptr;
    c->pos = d.rope ? nullptr : vecp("enc.pos_embed");
    c->rope = d.rope ? (float *)(arena + rope_off) : nullptr;
    c->normg = vecp("enc.norm.weight");
    c->normb = vecp("enc.norm.bias");
    c->layers.resize(d.depth);
    c->head_layers.resize(C > 0 ? d.head_blocks : 0);
    c->has_q = c->has_k = false;
    auto setup_layer = [&](Layer &L, const std::string &p) {
        L.qkv = c->by_name[p + "attn_qkv.weight"];
        L.out = c->by_name[p + "attn_out.weight"];
        L.up = c->by_name[p + "ffn_up.weight"];
        L.down = c->by_name[p + "ffn_down.weight"];
        L.ln1g = vecp(p + "ln1.weight"); L.ln1b = vecp(p + "ln1.bias");
        L.ln2g = vecp(p + "ln2.weight"); L.ln2b = vecp(p + "ln2.bias");
        L.bqkv = vecp(p + "attn_qkv.bias"); L.bout = vecp(p + "attn_out.bias");
        L.bup = vecp(p + "ffn_up.bias"); L.bdown = vecp(p + "ffn_down.bias");
    };
    for (int i = 0; i < d.depth; ++i) setup_layer(c->layers[i], "enc.blk." + std::to_string(i) + ".");
    for (size_t i = 0; i < c->head_layers.size(); ++i) setup_layer(c->head_layers[i], "head.blk." + std::to_string(i) + ".");
    if (C > 0) {
        Head &h = c->head;
        const std::string p = "head.xattn.";
        h.C = C; h.Cpad = Cpad;
        h.q0 = vecp("head.query_token");
        h.ln1g = vecp(p + "ln1.weight"); h.ln1b = vecp(p + "ln1.bias");
        h.ln2g = vecp(p + "ln2.weight"); h.ln2b = vecp(p + "ln2.bias");
        h.wq = c->by_name[p + "attn_q.weight"]; h.bq = vecp(p + "attn_q.bias");
        h.wk = c->by_name[p + "attn_k.weight"]; h.bk = vecp(p + "attn_k.bias");
        h.wv = c->by_name[p + "attn_v.weight"]; h.bv = vecp(p + "attn_v.bias");
        h.wo = c->by_name[p + "attn_out.weight"]; h.bo = vecp(p + "attn_out.bias");
        h.wup = c->by_name[p + "ffn_up.weight"]; h.bup = vecp(p + "ffn_up.bias");
        h.wdown = c->by_name[p + "ffn_down.weight"]; h.bdown = vecp(p + "ffn_down.bias");
        h.wc = c->by_name["head.classifier.weight"]; h.bc = vecp("head.classifier.bias");
        h.wc.ne1 = Cpad;   // the GEMM runs over the padded rows
    }
    for (auto &pr : expand_pairs(c)) {
        c->has_q |= is_block_dt(pr.first->dev_dt);
        c->has_k |= is_kquant_dt(pr.first->dev_dt);
    }
    if (hipEventCreate(&c->ev0) != hipSuccess || hipEventCreate(&c->ev1) != hipSuccess) {
        jepa_free(c);
        return fail(JEPA_E_HIP, "create: hipEventCreate failed");
    }
    c->have_events = true;
    {   // this device's copy of the no-allocation encode's scratch; a failure
        // here only matters to jepa_encode_noalloc, which looks it up again
        void *p = nullptr;
        if (scratch_address(&p) != hipSuccess) (void)hipGetLastError();
    }
    *out = c;
    return JEPA_OK;
}

static jepa_status gemm(jepa_ctx *c, int cls, hipStream_t s, int conc, const void *a, int64_t M, int64_t K,
                        const DevTensor &w, const float *bias, int epi, void *out, int64_t ldo,
                        float *kpart = nullptr) {
    GemmArgs g{};
    g.a = a; g.w = w.ptr; g.wscale = w.scale; g.bias = bias; g.out = out;
    g.M = M; g.N = w.ne1; g.K = K; g.lda = K; g.ldo = ldo;
    g.conc = conc;
    g.kpart = kpart;
    return launch(c, cls, s, [&] { return launch_gemm(c->act, w.dev_dt, epi, g, s); });
}

// Number of batch parts encoded concurrently, one HIP stream each.  Items
// are independent, so the parts share nothing but the weights: when one
// part's kernel is in its last, partial round of workgroups, another part's
// kernels fill the idle CUs (measured on MI355X, LeVJEPA ViT-L/16 batch 4:
// 14.5 ms with one part, 13.4 with two, 12.9 with four).  JEPA_STREAMS
// overrides the default of 4.
static int n_parts(const jepa_ctx *c, int batch) {
    int want = 4;
    if (const char *e = getenv("JEPA_STREAMS")) want = atoi(e);
    if (c->parts_set > 0) want = c->parts_set;
    want = std::max(1, std::min(want, jepa_ctx::MAX_PARTS));
    return std::min(want, batch);
}

// Part streams are non-blocking streams of default priority, ordered against
// the caller's stream by the fork / join events alone (blocking streams,
// which also order against the legacy NULL stream at every launch, measured
// slower than running the parts one after another).
static jepa_status ensure_streams(jepa_ctx *c, int parts) {
    if (parts < 2) return JEPA_OK;
    if (!c->fork_ev) HIP_TRY(hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming));
    for (int i = 0; i < parts - 1; ++i) {
        if (!c->aux[i]) HIP_TRY(hipStreamCreateWithFlags(&c->aux[i], hipStreamNonBlocking));
        if (!c->join_ev[i]) HIP_TRY(hipEventCreateWithFlags(&c->join_ev[i], hipEventDisableTiming));
    }
    return JEPA_OK;
}

// One pre-LN block on the rows of items b0 .. b0+nb-1 of the residual stream
// (row r0 = b0*N on), on stream s: LN1, the qkv GEMM (q scaled, optionally
// rotated; v to V^T), attention, out-projection + residual, LN2, fc1 + GELU,
// fc2 + residual.  expand: the q8_0 / q4_0 matrices' act-dtype copies.
static jepa_status run_block(jepa_ctx *c, const Ws &w, const Layer &L, bool expand, hipStream_t s, int conc,
                             int64_t r0, int b0, int nb, bool causal, const float *rope) {
    const jepa_dims &d = c->d;
    const int D = c->D, F = c->F, es = c->es, dh = D / c->H;
    auto rows = [&](void *base, int64_t first, int64_t width, int esz) {
        return (void *)((unsigned char *)base + first * width * esz);
    };
    const DevTensor &Wqkv = expand ? L.xqkv : L.qkv, &Wout = expand ? L.xout : L.out;
    const DevTensor &Wup = expand ? L.xup : L.up, &Wdown = expand ? L.xdown : L.down;
    const int64_t M = (int64_t)nb * c->N;
    float *x = (float *)rows(w.x, r0, D, 4);
    void *hn = rows(w.hn, r0, D, es), *qkv = rows(w.qkv, r0, 3 * D, es);
    void *o = rows(w.o, r0, D, es), *u = rows(w.u, r0, F, es);
    void *vt = rows(w.vt, b0, D * c->npad, es);
    AttnArgs aa{};
    aa.qk = qkv; aa.ld_qk = 3 * D; aa.vt = vt; aa.npad = c->npad;
    aa.out = o; aa.B = nb; aa.N = c->N; aa.heads = c->H;
    aa.has_cls = d.has_cls; aa.block_causal = causal; aa.per_slot = c->per_slot;
    aa.q_prescaled = 1;
    aa.dh = dh;
    aa.kvpart = w.kvpart ? w.kvpart + (size_t)KVSPLIT_MAX * r0 * c->H * (dh + 2) : nullptr;
    // the int8 path (jepa_set_int8_matmul) for q8_0 / q4_0 matrices: the
    // product's input is quantised per 32-block into this part's rows of
    // qa / qas (pitch K), then multiplied on int8 MFMA
    const bool i8 = c->int8_mm && !expand;
    const int64_t kf = std::max(D, F);
    int8_t *qa = i8 ? w.qa + r0 * kf : nullptr;
    float *qas = i8 ? w.qas + r0 * (kf / 32) : nullptr;
    auto run_gemm = [&](int cls, GemmArgs g, int w_dt, int epi) -> jepa_status {
        if (i8 && (w_dt == JEPA_Q8_0 || w_dt == JEPA_Q4_0)) {
            const void *in = g.a;
            const int64_t ld = g.lda;
            TRY(launch(c, K_QUANT_ACT, s, [&] { return launch_quant_act(c->act, in, ld, g.M, g.K, qa, g.K, qas, s); }));
            g.a = qa; g.lda = g.K; g.ascale = qas;
            return launch(c, cls, s, [&] { return launch_gemm_i8(c->act, w_dt, epi, g, s); });
        }
        return launch(c, cls, s, [&] { return launch_gemm(c->act, w_dt, epi, g, s); });
    };
    auto mm = [&](int cls, const void *a, int64_t K, const DevTensor &W, const float *bias, int epi, void *out,
                  int64_t ldo, float *kp) -> jepa_status {
        GemmArgs g{};
        g.a = a; g.w = W.ptr; g.wscale = W.scale; g.bias = bias; g.out = out;
        g.M = M; g.N = W.ne1; g.K = K; g.lda = K; g.ldo = ldo;
        g.conc = conc;
        g.kpart = kp;
        return run_gemm(cls, g, W.dev_dt, epi);
    };
    TRY(launch(c, K_LN, s, [&] { return launch_layernorm(x, M, D, L.ln1g, L.ln1b, d.ln_eps, hn, c->act, s); }));
    {   // q, k to qkv; v transposed straight into V^T
        GemmArgs g{};
        g.a = hn; g.w = Wqkv.ptr; g.wscale = Wqkv.scale; g.bias = L.bqkv; g.out = qkv;
        g.M = M; g.N = Wqkv.ne1; g.K = D; g.lda = D; g.ldo = 3 * D;
        g.ntok = c->N; g.vt = vt; g.npad = c->npad; g.vcol0 = 2 * D;
        g.rope = rope; g.head_dim = dh;
        g.qscale = attn_q_scale(dh);   // the softmax scale and base change, folded into q
        g.conc = conc;
        TRY(run_gemm(K_GEMM_QKV, g, Wqkv.dev_dt, EPI_QKV));
    }
    TRY(launch(c, K_ATTN, s, [&] { return launch_attention(c->act, aa, s); }));
    // f32 models: scratch for splitting the residual GEMMs' K (each batch
    // part its own rows of it)
    float *kpart = w.kpart ? w.kpart + (size_t)KSPLIT_MAX * r0 * D : nullptr;
    TRY(mm(K_GEMM_OUT, o, D, Wout, L.bout, EPI_RESID, x, D, kpart));
    TRY(launch(c, K_LN, s, [&] { return launch_layernorm(x, M, D, L.ln2g, L.ln2b, d.ln_eps, hn, c->act, s); }));
    TRY(mm(K_GEMM_FC1, hn, D, Wup, L.bup, EPI_GELU, u, F, nullptr));
    TRY(mm(K_GEMM_FC2, u, F, Wdown, L.bdown, EPI_RESID, x, D, kpart));
    return JEPA_OK;
}

// Whether the patch-embed GEMM can gather its A tile straight from these
// frames: a 16-bit act dtype, 8-byte runs of a patch row ((patch * 3) % 8
// == 0, rows of (img_w * 3) % 8 == 0 bytes, 8-byte aligned frames) and at
// most 256 8-element K chunks, 32-bit frame offsets.  Otherwise the frames go through the
// patchify kernel into the patch matrix first.
static bool implicit_patch(const jepa_ctx *c, const uint8_t *frames, int items) {
    const jepa_dims &d = c->d;
    return c->act != JEPA_F32 && (3 * d.patch) % 8 == 0 && (3 * d.img_w) % 8 == 0 &&
           ((uintptr_t)frames & 7) == 0 && c->Kp / 8 <= 256 &&
           (int64_t)items * d.frames * d.img_h * d.img_w * 3 < (1ll << 32);
}

// Items per batch part.  The GEMMs tile each part's rows in 256-row tiles,
// a last tile of at most 128 rows taking half a tile's time, so equal parts
// can leave most of a tile idle (32 images of 197 tokens in parts of 8: 1576
// rows, 6 tiles and 40 rows).  Among the splits whose part sizes differ by
// at most 2 items, the one with the fewest tile-times is taken (ties: the
// most even); 32 images -> 9, 9, 7, 7 measured 5.40 vs 5.50 ms on MI355X,
// while 9, 9, 9, 5 (fewer tiles, one short part) measured 5.72.
static void part_sizes(int batch, int parts, int64_t tokens, int *out) {
    auto tile_cost = [](int64_t rows) {   // in half tiles
        const int64_t full = rows / 256, rest = rows % 256;
        return 2 * full + (rest == 0 ? 0 : rest <= 128 ? 1 : 2);
    };
    const int base = batch / parts;
    int best[jepa_ctx::MAX_PARTS], cur[jepa_ctx::MAX_PARTS];
    for (int p = 0; p < parts; ++p) best[p] = base + (p < batch % parts ? 1 : 0);
    int64_t best_cost = 0, best_spread = 2;
    for (int p = 0; p < parts; ++p) best_cost += tile_cost(best[p] * tokens);
    best_spread = best[0] - best[parts - 1];
    // part sizes in [lo, lo + 2], non-increasing, summing to batch
    for (int lo = base - 1; lo <= base; ++lo) {
        if (lo < 1) continue;
        const std::function<void(int, int)> rec = [&](int p, int left) {
            if (p == parts) {
                if (left) return;
                int64_t cost = 0;
                for (int i = 0; i < parts; ++i) cost += tile_cost(cur[i] * tokens);
                const int spread = cur[0] - cur[parts - 1];
                if (cost < best_cost || (cost == best_cost && spread < best_spread)) {
                    best_cost = cost;
                    best_spread = spread;
                    for (int i = 0; i < parts; ++i) best[i] = cur[i];
                }
                return;
            }
            for (int v = (p ? cur[p - 1] : lo + 2); v >= lo; --v) {
                if (v > left) continue;
                cur[p] = v;
                rec(p + 1, left - v);
            }
        };
        rec(0, batch);
    }
    for (int p = 0; p < parts; ++p) out[p] = best[p];
}

// The launch sequence of one encode of `batch` items with device frames fr
// into the token map Y, over the buffers w, in `parts` concurrent parts
// (part 0 on s0, the others on the context's internal streams, forked from
// and joined back onto s0).  expand: the block matrices' act-dtype copies
// (already written on s0).  Whatever it returns, the parts are joined back
// onto s0, so that no part's work outlives the caller's stream order.
static jepa_status encode_parts(jepa_ctx *c, const Ws &w, const uint8_t *fr, int batch, float *Y, hipStream_t s0,
                                int parts, bool expand) {
    const jepa_dims &d = c->d;
    const size_t frame_bytes = (size_t)d.frames * d.img_h * d.img_w * 3;   // per item
    if (parts > 1) {
        HIP_TRY(hipEventRecord(c->fork_ev, s0));
        for (int p = 1; p < parts; ++p) HIP_TRY(hipStreamWaitEvent(c->aux[p - 1], c->fork_ev, 0));
    }

    // part p: items [b0, b0 + nb), its own stream and row ranges of every buffer
    struct Part {
        hipStream_t s;
        int b0, nb;
        int64_t r0, M;
    };
    Part P[jepa_ctx::MAX_PARTS];
    int sizes[jepa_ctx::MAX_PARTS];
    part_sizes(batch, parts, c->N, sizes);
    for (int p = 0, b = 0; p < parts; ++p) {
        const int nb = sizes[p];
        P[p] = Part{p == 0 ? s0 : c->aux[p - 1], b, nb, (int64_t)b * c->N, (int64_t)nb * c->N};
        b += nb;
    }
    const int D = c->D, es = c->es;
    auto rows = [&](void *base, int64_t r0, int64_t width, int esz) {
        return (void *)((unsigned char *)base + r0 * width * esz);
    };

    auto body = [&]() -> jepa_status {
    for (int p = 0; p < parts; ++p) {
        const Part &q = P[p];
        const uint8_t *qf = fr + (size_t)q.b0 * frame_bytes;
        GemmArgs g{};
        g.w = c->wpe.ptr; g.bias = c->bpe; g.out = rows(w.x, q.r0, D, 4);
        g.M = (int64_t)q.nb * c->Np; g.N = D; g.K = c->Kp; g.lda = c->Kp; g.ldo = D;
        g.pos = c->pos; g.np = c->Np; g.ntok = c->N; g.has_cls = d.has_cls;
        if (implicit_patch(c, qf, q.nb)) {
            // the GEMM gathers and normalises its A tile from the frames
            g.a = nullptr;
            g.frames = qf; g.fT = d.frames; g.fH = d.img_h; g.fW = d.img_w; g.tubelet = d.tubelet;
            g.patch = d.patch; g.patch_len = c->P;
            for (int i = 0; i < 3; ++i) { g.pix_scale[i] = c->pix_scale[i]; g.pix_shift[i] = c->pix_shift[i]; }
        } else {
            PatchifyArgs pa{};
            pa.frames = qf; pa.B = q.nb; pa.T = d.frames; pa.H = d.img_h; pa.W = d.img_w;
            pa.tubelet = d.tubelet; pa.patch = d.patch;
            for (int i = 0; i < 3; ++i) { pa.mean[i] = d.mean[i]; pa.std[i] = d.std[i]; }
            pa.out = rows(w.patch, (int64_t)q.b0 * c->Np, c->Kp, es); pa.ld = c->Kp;
            TRY(launch(c, K_PATCHIFY, q.s, [&] { return launch_patchify(c->act, pa, q.s); }));
            g.a = pa.out;
        }
        TRY(launch(c, K_GEMM_PATCH, q.s, [&] { return launch_gemm(c->act, c->act, EPI_PATCH, g, q.s); }));
        if (d.has_cls)
            TRY(launch(c, K_CLS_ROWS, q.s, [&] {
                return launch_cls_rows((float *)g.out, c->cls, c->pos, q.nb, c->N, D, q.s);
            }));
    }

    for (int i = 0; i < c->L; ++i)
        for (int p = 0; p < parts; ++p)
            TRY(run_block(c, w, c->layers[i], expand, P[p].s, parts, P[p].r0, P[p].b0, P[p].nb,
                          d.mask == JEPA_MASK_BLOCK_CAUSAL, c->rope));
    for (int p = 0; p < parts; ++p) {
        const Part &q = P[p];
        float *x = (float *)rows(w.x, q.r0, D, 4);
        float *y = Y + q.r0 * D;
        TRY(launch(c, K_FINAL_LN, q.s, [&] {
            return launch_layernorm(x, q.M, D, c->normg, c->normb, d.ln_eps, y, JEPA_F32, q.s);
        }));
    }
    return JEPA_OK;
    };
    const jepa_status st = body();
    for (int p = 1; p < parts; ++p) {
        HIP_TRY(hipEventRecord(c->join_ev[p - 1], c->aux[p - 1]));
        HIP_TRY(hipStreamWaitEvent(s0, c->join_ev[p - 1], 0));
    }
    return st;
}

static jepa_status check_encode_args(const jepa_ctx *c, const uint8_t *frames, int batch) {
    if (!c || !frames) return fail(JEPA_E_INVALID_ARG, "encode: null argument");
    if (batch <= 0) return fail(JEPA_E_INVALID_ARG, "encode: batch must be > 0 (got %d)", batch);
    if ((int64_t)batch * c->N > (int64_t)65535 * 128)
        return fail(JEPA_E_UNSUPPORTED, "encode: batch*tokens %lld too large", (long long)batch * c->N);
    return JEPA_OK;
}

jepa_status jepa_encode_noalloc(jepa_ctx *c, const uint8_t *frames, int batch, float *tokens_out,
                                void *hip_stream) {
    TRY(check_encode_args(c, frames, batch));
    if (!tokens_out) return fail(JEPA_E_INVALID_ARG, "encode_noalloc: tokens_out is required");
    if (c->has_k)
        return fail(JEPA_E_UNSUPPORTED, "encode_noalloc: K-quant matrices run from an expanded copy that "
                    "jepa_encode allocates");
    c->encoded = false;
    c->last_tokens = nullptr;
    c->last_batch = 0;
    const WsLayout lay = ws_layout(c, batch, false);
    if (lay.total > JEPA_NOALLOC_SCRATCH_BYTES)
        return fail(JEPA_E_OOM, "encode_noalloc: batch %d needs %zu bytes of buffers; the static scratch holds %zu",
                    batch, lay.total, (size_t)JEPA_NOALLOC_SCRATCH_BYTES);
    void *base = nullptr;
    const hipError_t e = scratch_address(&base);
    if (e != hipSuccess) return fail(JEPA_E_HIP, "encode_noalloc: address of the static scratch: %s", hipGetErrorString(e));
    const Ws w = ws_pointers(c, lay, (unsigned char *)base);
    hipStream_t s = (hipStream_t)hip_stream;
    // the last key tile of each head reads V^T's padding columns: finite
    // values, cleared by a kernel (the array holds whatever the last call left)
    const int64_t vt_words = (int64_t)batch * c->D * c->npad * c->es / 4;
    const hipError_t fe = launch_fill((float *)w.vt, vt_words, 0.f, s);
    if (fe != hipSuccess) return fail(JEPA_E_HIP, "encode_noalloc: clearing V^T: %s", hipGetErrorString(fe));
    // no timing events (they are created on demand)
    const uint32_t prof = c->prof;
    c->prof = 0;
    const jepa_status st = encode_parts(c, w, frames, batch, tokens_out, s, 1, false);
    c->prof = prof;
    return st;
}

jepa_status jepa_encode(jepa_ctx *c, const uint8_t *frames, int batch, int frames_on_device,
                        float *tokens_out, void *hip_stream) {
    TRY(check_encode_args(c, frames, batch));
    // pool / classify read nothing of a failed encode, nor of the previous
    // one once this call has started (its workspace may be reallocated)
    c->encoded = false;
    c->last_tokens = nullptr;
    c->last_batch = 0;
    TRY(ensure_workspace(c, batch));
    const int parts = n_parts(c, batch);
    TRY(ensure_streams(c, parts));
    hipStream_t s0 = (hipStream_t)hip_stream;
    const jepa_dims &d = c->d;
    const uint8_t *fr = frames;
    if (!frames_on_device) {
        // copy into the pinned staging buffer (once the previous copy out of
        // it has finished), then DMA to the device on the caller's stream:
        // the call returns after enqueue and the caller's buffer is free
        const size_t bytes = (size_t)batch * d.frames * d.img_h * d.img_w * 3;
        if (c->h_pending) HIP_TRY(hipEventSynchronize(c->h_ev));
        c->h_pending = false;
        if (bytes > c->h_frames_bytes) {
            if (c->h_frames) HIP_TRY(hipHostFree(c->h_frames));
            c->h_frames = nullptr;
            c->h_frames_bytes = 0;
            if (hipHostMalloc((void **)&c->h_frames, bytes, hipHostMallocDefault) != hipSuccess) {
                c->h_frames = nullptr;
                (void)hipGetLastError();
                return fail(JEPA_E_OOM, "encode: pinned staging of %zu frame bytes failed", bytes);
            }
            c->h_frames_bytes = bytes;
        }
        if (!c->h_ev) HIP_TRY(hipEventCreateWithFlags(&c->h_ev, hipEventDisableTiming));
        memcpy(c->h_frames, frames, bytes);
        HIP_TRY(hipMemcpyAsync(c->w.frames, c->h_frames, bytes, hipMemcpyHostToDevice, s0));
        HIP_TRY(hipEventRecord(c->h_ev, s0));
        c->h_pending = true;
        fr = c->w.frames;
    }
    float *Y = tokens_out ? tokens_out : c->w.y;
    HIP_TRY(hipEventRecord(c->ev0, s0));
    const bool expand = use_expand(c, batch, parts);
    c->last_expand = expand;
    if (expand) {
        TRY(ensure_expanded(c));
        if (!c->x_written) {
            if (!c->x_ev) HIP_TRY(hipEventCreateWithFlags(&c->x_ev, hipEventDisableTiming));
            TRY(launch(c, K_EXPAND, s0, [&] { return launch_expand(c->act, c->xjobs, c->n_xjobs, c->x_nblk, s0); }));
            HIP_TRY(hipEventRecord(c->x_ev, s0));
            c->x_written = true;
        } else {
            // written by an earlier encode, possibly on another stream
            HIP_TRY(hipStreamWaitEvent(s0, c->x_ev, 0));
        }
    }
    TRY(encode_parts(c, c->w, fr, batch, Y, s0, parts, expand));
    HIP_TRY(hipEventRecord(c->ev1, s0));
    c->last_tokens = Y;
    c->last_batch = batch;
    c->encoded = true;
    return JEPA_OK;
}

jepa_status jepa_classify(jepa_ctx *c, float *logits_out, void *hip_stream) {
    if (!c || !logits_out) return fail(JEPA_E_INVALID_ARG, "classify: null argument");
    if (c->head.C <= 0) return fail(JEPA_E_UNSUPPORTED, "classify: the model has no classifier head");
    if (!c->encoded) return fail(JEPA_E_STATE, "classify: no encode yet");
    if (c->N > XATTN_MAX_N) return fail(JEPA_E_UNSUPPORTED, "classify: %d tokens exceed %d", c->N, XATTN_MAX_N);
    const jepa_dims &d = c->d;
    const Head &h = c->head;
    const bool xp = c->last_expand;   // the block matrices' copies are current
    const DevTensor &wq = xp ? h.xwq : h.wq, &wk = xp ? h.xwk : h.wk, &wv = xp ? h.xwv : h.wv;
    const DevTensor &wo = xp ? h.xwo : h.wo, &wup = xp ? h.xwup : h.wup, &wdown = xp ? h.xwdown : h.wdown;
    hipStream_t s = (hipStream_t)hip_stream;
    const int B = c->last_batch, D = c->D, F = c->F, dh = D / c->H;
    const int64_t M = (int64_t)B * c->N;
    // the head's blocks run on the residual stream, seeded with the token map
    HIP_TRY(hipMemcpyAsync(c->w.x, c->last_tokens, (size_t)M * D * 4, hipMemcpyDeviceToDevice, s));
    for (const Layer &L : c->head_layers) TRY(run_block(c, c->w, L, c->last_expand, s, 1, 0, 0, B, false, nullptr));
    // keys and values of the normalised tokens (in the qkv buffer, pitch 3D)
    TRY(launch(c, K_LN, s, [&] { return launch_layernorm(c->w.x, M, D, h.ln1g, h.ln1b, d.ln_eps, c->w.hn, c->act, s); }));
    unsigned char *kv = (unsigned char *)c->w.qkv;
    TRY(gemm(c, K_HEAD, s, 1, c->w.hn, M, D, wk, h.bk, EPI_STORE, kv, 3 * D));
    TRY(gemm(c, K_HEAD, s, 1, c->w.hn, M, D, wv, h.bv, EPI_STORE, kv + (size_t)D * c->es, 3 * D));
    // the query row of every item: W_q q0 + b_q
    TRY(launch(c, K_HEAD, s, [&] { return launch_cls_rows(c->w.hx, h.q0, nullptr, B, 1, D, s); }));
    TRY(launch(c, K_HEAD, s, [&] { return launch_cast(c->w.hx, (int64_t)B * D, c->w.hh, c->act, s); }));
    TRY(gemm(c, K_HEAD, s, 1, c->w.hh, B, D, wq, h.bq, EPI_STORE, c->w.hq, D));
    TRY(launch(c, K_HEAD, s, [&] {
        return launch_xattn(c->act, c->w.hq, kv, kv + (size_t)D * c->es, 3 * D, B, c->N, c->H, dh, c->w.ho, s);
    }));
    // x = q0 + out_proj(o); x += MLP(LN2 x); scores = W_c x + b_c
    TRY(gemm(c, K_HEAD, s, 1, c->w.ho, B, D, wo, h.bo, EPI_RESID, c->w.hx, D));
    TRY(launch(c, K_HEAD, s, [&] { return launch_layernorm(c->w.hx, B, D, h.ln2g, h.ln2b, d.ln_eps, c->w.hh, c->act, s); }));
    TRY(gemm(c, K_HEAD, s, 1, c->w.hh, B, D, wup, h.bup, EPI_GELU, c->w.hu, F));
    TRY(gemm(c, K_HEAD, s, 1, c->w.hu, B, F, wdown, h.bdown, EPI_RESID, c->w.hx, D));
    TRY(launch(c, K_HEAD, s, [&] { return launch_cast(c->w.hx, (int64_t)B * D, c->w.hh, c->act, s); }));
    TRY(launch(c, K_HEAD, s, [&] { return launch_fill(c->w.hl, (int64_t)B * h.Cpad, 0.f, s); }));
    TRY(gemm(c, K_HEAD, s, 1, c->w.hh, B, D, h.wc, h.bc, EPI_RESID, c->w.hl, h.Cpad));
    HIP_TRY(hipMemcpy2DAsync(logits_out, (size_t)h.C * 4, c->w.hl, (size_t)h.Cpad * 4, (size_t)h.C * 4, B,
                             hipMemcpyDeviceToDevice, s));
    return JEPA_OK;
}

jepa_status jepa_set_batch_parts(jepa_ctx *c, int parts) {
    if (!c) return fail(JEPA_E_INVALID_ARG, "set_batch_parts: null context");
    if (parts < 0 || parts > jepa_ctx::MAX_PARTS)
        return fail(JEPA_E_INVALID_ARG, "set_batch_parts: parts must be in [0, %d] (got %d)", jepa_ctx::MAX_PARTS,
                    parts);
    c->parts_set = parts;
    return JEPA_OK;
}

jepa_status jepa_set_int8_matmul(jepa_ctx *c, int enable) {
    if (!c) return fail(JEPA_E_INVALID_ARG, "set_int8_matmul: null context");
    if (enable != 0 && enable != 1) return fail(JEPA_E_INVALID_ARG, "set_int8_matmul: enable must be 0 or 1");
    if (enable && c->act == JEPA_F32) return fail(JEPA_E_UNSUPPORTED, "set_int8_matmul: f32 models have no block matrices");
    if (enable && c->has_k)
        return fail(JEPA_E_UNSUPPORTED, "set_int8_matmul: K-quant models run from their expanded act-dtype copies");
    if (enable && (c->D % 128 || c->F % 128))
        return fail(JEPA_E_UNSUPPORTED, "set_int8_matmul: dim and mlp_dim must be multiples of 128");
    if ((bool)enable == c->int8_mm) return JEPA_OK;
    // the workspace layout changes: the next encode allocates it again
    TRY(release_workspace(c));
    c->int8_mm = enable != 0;
    return JEPA_OK;
}

jepa_status jepa_pool(jepa_ctx *c, int mode, float *out, void *hip_stream) {
    if (!c || !out) return fail(JEPA_E_INVALID_ARG, "pool: null argument");
    if (!c->encoded) return fail(JEPA_E_STATE, "pool: nothing encoded yet");
    hipStream_t s = (hipStream_t)hip_stream;
    const int B = c->last_batch;
    switch (mode) {
        case JEPA_POOL_CLS:
            if (!c->d.has_cls) return fail(JEPA_E_STATE, "pool: the model has no CLS token");
            return launch(c, K_POOL, s, [&] { return launch_pool_cls(c->last_tokens, B, c->N, c->D, out, s); });
        case JEPA_POOL_MEAN:
            return launch(c, K_POOL, s, [&] { return launch_pool_mean(c->last_tokens, B, c->N, c->D, c->d.has_cls, c->w.pool, out, s); });
        case JEPA_POOL_NONE:   // a kernel, so that the copy is ordered on the compute queue like the rest
            return launch(c, K_POOL, s, [&] { return launch_copy_f32(c->last_tokens, (int64_t)B * c->N * c->D, out, s); });
    }
    return fail(JEPA_E_INVALID_ARG, "pool: unknown mode %d", mode);
}

void jepa_free(jepa_ctx *c) {
    if (!c) return;
    (void)hipDeviceSynchronize();
    if (c->arena) (void)hipFree(c->arena);
    if (c->ws) (void)hipFree(c->ws);
    if (c->xbuf) (void)hipFree(c->xbuf);
    if (c->h_frames) (void)hipHostFree(c->h_frames);
    if (c->h_ev) (void)hipEventDestroy(c->h_ev);
    if (c->x_ev) (void)hipEventDestroy(c->x_ev);
    if (c->have_events) {
        (void)hipEventDestroy(c->ev0);
        (void)hipEventDestroy(c->ev1);
    }
    if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
    for (int i = 0; i < jepa_ctx::MAX_PARTS - 1; ++i) {
        if (c->join_ev[i]) (void)hipEventDestroy(c->join_ev[i]);
        if (c->aux[i]) (void)hipStreamDestroy(c->aux[i]);
    }
    for (auto &r : c->pending) {
        if (r.a) (void)hipEventDestroy(r.a);
        if (r.b) (void)hipEventDestroy(r.b);
    }
    for (auto e : c->event_pool) (void)hipEventDestroy(e);
    delete c;
}

float jepa_last_compute_ms(jepa_ctx *c) {
    if (!c || !c->encoded) return -1.f;
    if (hipEventSynchronize(c->ev1) != hipSuccess) return -1.f;
    float ms = -1.f;
    if (hipEventElapsedTime(&ms, c->ev0, c->ev1) != hipSuccess) return -1.f;
    return ms;
}

size_t jepa_model_n_bytes(const jepa_ctx *c) { return c ? c->model_bytes : 0; }
size_t jepa_device_weight_bytes(const jepa_ctx *c) { return c ? c->arena_bytes : 0; }
size_t jepa_workspace_bytes(const jepa_ctx *c, int batch) {
    if (!c || batch <= 0) return 0;
    return ws_layout(c, batch).total + (use_expand(c, batch, n_parts(c, batch)) ? expand_bytes(c) : 0);
}

jepa_status jepa_dequant_tensor(jepa_ctx *c, const char *name, float *out_dev, void *hip_stream) {
    if (!c || !name || !out_dev) return fail(JEPA_E_INVALID_ARG, "dequant: null argument");
    auto it = c->by_name.find(name);
    if (it == c->by_name.end()) return fail(JEPA_E_MISSING_TENSOR, "dequant: no tensor '%s'", name);
    const DevTensor &t = it->second;
    hipStream_t s = (hipStream_t)hip_stream;
    // the patch-embed matrix is stored with padded rows; copy row by row
    if (std::string(name) == "enc.patch_embed.weight" && c->Kp != t.ne0) {
        for (int64_t r = 0; r < t.ne1; ++r) {
            hipError_t e = launch_dequant(t.dev_dt, (const unsigned char *)t.ptr + r * c->Kp * c->es,
                                          nullptr, nullptr, 1, t.ne0, out_dev + r * t.ne0, s);
            if (e != hipSuccess) return fail(JEPA_E_HIP, "dequant: %s", hipGetErrorString(e));
        }
        return JEPA_OK;
    }
    hipError_t e = launch_dequant(t.dev_dt, t.ptr, t.scale, t.sub, t.ne1, t.ne0, out_dev, s);
    if (e != hipSuccess) return fail(JEPA_E_HIP, "dequant: %s", hipGetErrorString(e));
    return JEPA_OK;
}

jepa_status jepa_set_profiling(jepa_ctx *c, uint32_t class_mask) {
    if (!c) return fail(JEPA_E_INVALID_ARG, "set_profiling: null context");
    c->prof = class_mask;
    return JEPA_OK;
}

int jepa_kernel_stats(jepa_ctx *c, jepa_kernel_stat *out, int cap) {
    if (!c) return fail(JEPA_E_INVALID_ARG, "kernel_stats: null context");
    for (auto &r : c->pending) {
        if (hipEventSynchronize(r.b) != hipSuccess) return fail(JEPA_E_HIP, "kernel_stats: event sync failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(JEPA_E_HIP, "kernel_stats: elapsed failed");
        c->stat_launches[r.cls] += 1;
        c->stat_ms[r.cls] += ms;
        c->event_pool.push_back(r.a);
        c->event_pool.push_back(r.b);
    }
    c->pending.clear();
    for (int i = 0; i < K_COUNT && i < cap; ++i) {
        out[i].name = kClassNames[i];
        out[i].launches = c->stat_launches[i];
        out[i].total_ms = c->stat_ms[i];
    }
    return K_COUNT;
}

void jepa_reset_kernel_stats(jepa_ctx *c) {
    if (!c) return;
    jepa_kernel_stat tmp[K_COUNT];
    (void)jepa_kernel_stats(c, tmp, K_COUNT);
    for (int i = 0; i < K_COUNT; ++i) { c->stat_launches[i] = 0; c->stat_ms[i] = 0.0; }
}

// ---------------------------------------------------------------------------
// single kernels (include/jepa_mi355x_ops.h)
// ---------------------------------------------------------------------------

static jepa_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return JEPA_OK;
    if (e == hipErrorInvalidValue) return fail(JEPA_E_SHAPE, "%s: shape or argument outside the kernel's contract", what);
    return fail(JEPA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool act_ok(int dt) { return dt == JEPA_F32 || dt == JEPA_F16 || dt == JEPA_BF16; }

jepa_status jepa_op_patchify(int act_dtype, const uint8_t *frames, int batch, int frames_per_item,
                             int img_h, int img_w, int tubelet, int patch, const float mean[3],
                             const float std[3], void *out, int64_t ld, void *hip_stream) {
    if (!frames || !out || !mean || !std) return fail(JEPA_E_INVALID_ARG, "op_patchify: null argument");
    if (!act_ok(act_dtype)) return fail(JEPA_E_DTYPE, "op_patchify: bad act dtype");
    PatchifyArgs a{};
    a.frames = frames; a.B = batch; a.T = frames_per_item; a.H = img_h; a.W = img_w;
    a.tubelet = tubelet; a.patch = patch; a.out = out; a.ld = ld;
    for (int i = 0; i < 3; ++i) { a.mean[i] = mean[i]; a.std[i] = std[i]; }
    return hip_status(launch_patchify(act_dtype, a, (hipStream_t)hip_stream), "op_patchify");
}

jepa_status jepa_op_layernorm(const float *x, int64_t rows, int dim, const float *gamma,
                              const float *beta, float eps, void *y, int y_dtype, void *hip_stream) {
    if (!x || !gamma || !beta || !y) return fail(JEPA_E_INVALID_ARG, "op_layernorm: null argument");
    if (!act_ok(y_dtype)) return fail(JEPA_E_DTYPE, "op_layernorm: bad output dtype");
    return hip_status(launch_layernorm(x, rows, dim, gamma, beta, eps, y, y_dtype, (hipStream_t)hip_stream),
                      "op_layernorm");
}

jepa_status jepa_op_gemm(int act_dtype, const void *a, int64_t M, int64_t K, const void *w,
                         int w_dtype, const uint16_t *w_scale, int64_t N, const float *bias,
                         int epilogue, void *out, int64_t ldo, void *hip_stream) {
    if (!a || !w || !bias || !out) return fail(JEPA_E_INVALID_ARG, "op_gemm: null argument");
    if (!act_ok(act_dtype)) return fail(JEPA_E_DTYPE, "op_gemm: bad act dtype");
    if (epilogue < JEPA_EPI_STORE || epilogue > JEPA_EPI_RESID)
        return fail(JEPA_E_INVALID_ARG, "op_gemm: unknown epilogue %d", epilogue);
    GemmArgs g{};
    g.a = a; g.w = w; g.wscale = w_scale; g.bias = bias; g.out = out;
    g.M = M; g.N = N; g.K = K; g.lda = K; g.ldo = ldo;
    return hip_status(launch_gemm(act_dtype, w_dtype, epilogue, g, (hipStream_t)hip_stream), "op_gemm");
}

jepa_status jepa_op_quantize_act(int act_dtype, const void *x, int64_t rows, int64_t k, int8_t *codes_out,
                                 float *scales_out, void *hip_stream) {
    if (!x || !codes_out || !scales_out) return fail(JEPA_E_INVALID_ARG, "op_quantize_act: null argument");
    if (act_dtype != JEPA_F16 && act_dtype != JEPA_BF16) return fail(JEPA_E_DTYPE, "op_quantize_act: act must be F16 or BF16");
    if (rows <= 0 || k <= 0 || k % 32) return fail(JEPA_E_SHAPE, "op_quantize_act: rows > 0 and k a multiple of 32 required");
    return hip_status(launch_quant_act(act_dtype, x, k, rows, k, codes_out, k, scales_out, (hipStream_t)hip_stream),
                      "op_quantize_act");
}

jepa_status jepa_op_gemm_i8(int act_dtype, const int8_t *a_codes, const float *a_scales, int64_t M, int64_t K,
                            const void *w, int w_dtype, const uint16_t *w_scale, int64_t N, const float *bias,
                            int epilogue, void *out, int64_t ldo, void *hip_stream) {
    if (!a_codes || !a_scales || !w || !w_scale || !bias || !out) return fail(JEPA_E_INVALID_ARG, "op_gemm_i8: null argument");
    if (act_dtype != JEPA_F16 && act_dtype != JEPA_BF16) return fail(JEPA_E_DTYPE, "op_gemm_i8: act must be F16 or BF16");
    if (w_dtype != JEPA_Q8_0 && w_dtype != JEPA_Q4_0) return fail(JEPA_E_DTYPE, "op_gemm_i8: weights must be Q8_0 or Q4_0");
    if (epilogue < JEPA_EPI_STORE || epilogue > JEPA_EPI_RESID)
        return fail(JEPA_E_INVALID_ARG, "op_gemm_i8: unknown epilogue %d", epilogue);
    GemmArgs g{};
    g.a = a_codes; g.ascale = a_scales; g.w = w; g.wscale = w_scale; g.bias = bias; g.out = out;
    g.M = M; g.N = N; g.K = K; g.lda = K; g.ldo = ldo;
    return hip_status(launch_gemm_i8(act_dtype, w_dtype, epilogue, g, (hipStream_t)hip_stream), "op_gemm_i8");
}

jepa_status jepa_op_patch_embed(int act_dtype, const uint8_t *frames, int B, int T, int H, int W, int tubelet,
                                int patch, const float *mean, const float *std, const void *w, int64_t k_pitch,
                                int64_t n, const float *bias, const float *pos, int has_cls, float *out,
                                void *hip_stream) {
    if (!frames || !mean || !std || !w || !bias || !out) return fail(JEPA_E_INVALID_ARG, "op_patch_embed: null argument");
    if (act_dtype != JEPA_F16 && act_dtype != JEPA_BF16) return fail(JEPA_E_DTYPE, "op_patch_embed: act must be F16 or BF16");
    if (B <= 0 || T <= 0 || H <= 0 || W <= 0 || tubelet <= 0 || patch <= 0 || (has_cls != 0 && has_cls != 1) ||
        H % patch || W % patch || T % tubelet)
        return fail(JEPA_E_SHAPE, "op_patch_embed: bad shape");
    GemmArgs g{};
    g.w = w; g.bias = bias; g.out = out; g.pos = pos;
    g.np = (T / tubelet) * (H / patch) * (W / patch);
    g.ntok = g.np + has_cls; g.has_cls = has_cls;
    g.M = (int64_t)B * g.np; g.N = n; g.K = k_pitch; g.lda = k_pitch; g.ldo = n;
    g.frames = frames; g.fT = T; g.fH = H; g.fW = W; g.tubelet = tubelet; g.patch = patch;
    g.patch_len = tubelet * patch * patch * 3;
    for (int i = 0; i < 3; ++i) {
        if (!(std[i] > 0.f)) return fail(JEPA_E_INVALID_ARG, "op_patch_embed: std must be > 0");
        g.pix_scale[i] = (float)(1.0 / (255.0 * (double)std[i]));
        g.pix_shift[i] = (float)(-(double)mean[i] / (double)std[i]);
    }
    return hip_status(launch_gemm(act_dtype, act_dtype, EPI_PATCH, g, (hipStream_t)hip_stream), "op_patch_embed");
}

jepa_status jepa_op_gemm_qkv(int act_dtype, const void *a, int64_t M, int64_t K, const void *w,
                             int w_dtype, const uint16_t *w_scale, int heads, int head_dim,
                             const float *bias, int n_tokens, void *qk_out, int64_t ld_qk, void *vt,
                             int64_t npad, const float *rope, float q_scale, void *hip_stream) {
    if (!a || !w || !bias || !qk_out || !vt) return fail(JEPA_E_INVALID_ARG, "op_gemm_qkv: null argument");
    if (!act_ok(act_dtype)) return fail(JEPA_E_DTYPE, "op_gemm_qkv: bad act dtype");
    if (heads <= 0 || n_tokens <= 0) return fail(JEPA_E_INVALID_ARG, "op_gemm_qkv: heads and n_tokens must be > 0");
    if (head_dim != 32 && head_dim != 64) return fail(JEPA_E_UNSUPPORTED, "op_gemm_qkv: head_dim must be 32 or 64");
    GemmArgs g{};
    g.a = a; g.w = w; g.wscale = w_scale; g.bias = bias; g.out = qk_out;
    g.M = M; g.N = 3 * (int64_t)heads * head_dim; g.K = K; g.lda = K; g.ldo = ld_qk;
    g.ntok = n_tokens; g.vt = vt; g.npad = npad; g.vcol0 = 2 * (int64_t)heads * head_dim;
    g.rope = rope; g.head_dim = head_dim;
    g.qscale = q_scale == 1.f ? 0.f : q_scale;
    return hip_status(launch_gemm(act_dtype, w_dtype, EPI_QKV, g, (hipStream_t)hip_stream), "op_gemm_qkv");
}

jepa_status jepa_op_attention(int act_dtype, const void *qk, int64_t ld_qk, const void *vt,
                              int64_t npad, int batch, int n_tokens, int heads, int head_dim,
                              int has_cls, int mask, int tokens_per_slot, int q_prescaled,
                              void *out, void *hip_stream) {
    if (!qk || !vt || !out) return fail(JEPA_E_INVALID_ARG, "op_attention: null argument");
    if (!act_ok(act_dtype)) return fail(JEPA_E_DTYPE, "op_attention: bad act dtype");
    if (mask != JEPA_MASK_BIDIR && mask != JEPA_MASK_BLOCK_CAUSAL)
        return fail(JEPA_E_INVALID_ARG, "op_attention: unknown mask %d", mask);
    AttnArgs a{};
    a.qk = qk; a.ld_qk = ld_qk; a.vt = vt; a.npad = npad;
    a.out = out; a.B = batch; a.N = n_tokens; a.heads = heads;
    a.has_cls = has_cls ? 1 : 0; a.block_causal = mask == JEPA_MASK_BLOCK_CAUSAL;
    a.per_slot = tokens_per_slot;
    a.q_prescaled = q_prescaled ? 1 : 0;
    a.dh = head_dim;
    if (head_dim != 32 && head_dim != 64) return fail(JEPA_E_UNSUPPORTED, "op_attention: head_dim must be 32 or 64");
    return hip_status(launch_attention(act_dtype, a, (hipStream_t)hip_stream), "op_attention");
}

jepa_status jepa_op_transpose_v(int act_dtype, const void *qkv, int batch, int n_tokens,
                                int heads, int head_dim, void *vt, int64_t npad, void *hip_stream) {
    if (!qkv || !vt) return fail(JEPA_E_INVALID_ARG, "op_transpose_v: null argument");
    if (!act_ok(act_dtype)) return fail(JEPA_E_DTYPE, "op_transpose_v: bad act dtype");
    if (heads <= 0 || (head_dim != 32 && head_dim != 64))
        return fail(JEPA_E_UNSUPPORTED, "op_transpose_v: head_dim must be 32 or 64");
    return hip_status(launch_transpose_v(act_dtype, qkv, batch, n_tokens, heads * head_dim, vt, npad,
                                         (hipStream_t)hip_stream), "op_transpose_v");
}

jepa_status jepa_pack_blocks(int dtype, const uint8_t *blocks, int64_t rows, int64_t cols,
                             uint8_t *codes, uint16_t *scales) {
    if (!blocks || !codes || !scales || rows <= 0 || cols <= 0)
        return fail(JEPA_E_INVALID_ARG, "pack_blocks: bad arguments");
    if (dtype != JEPA_Q8_0 && dtype != JEPA_Q4_0) return fail(JEPA_E_DTYPE, "pack_blocks: dtype must be Q8_0 or Q4_0");
    if (cols % 32) return fail(JEPA_E_SHAPE, "pack_blocks: cols not a multiple of 32");
    pack_blocks(dtype, blocks, rows * (cols / 32), codes, scales);
    return JEPA_OK;
}

jepa_status jepa_op_mfma_i8_probe(int workgroups, int iters, int mode, float *out, void *hip_stream) {
    if (!out || workgroups <= 0 || iters <= 0 || mode < 0 || mode > 2)
        return fail(JEPA_E_INVALID_ARG, "op_mfma_i8_probe: bad arguments");
    return hip_status(launch_mfma_i8_probe(workgroups, iters, mode, out, (hipStream_t)hip_stream), "op_mfma_i8_probe");
}

jepa_status jepa_op_mfma_probe(int workgroups, int iters, int operands, float *out, void *hip_stream) {
    if (!out || workgroups <= 0 || iters <= 0 || operands < 0 || operands > 1)
        return fail(JEPA_E_INVALID_ARG, "op_mfma_probe: bad arguments");
    return hip_status(launch_mfma_probe(workgroups, iters, operands, out, (hipStream_t)hip_stream), "op_mfma_probe");
}

jepa_status jepa_rope_table(const jepa_dims *dims, float *out) {
    if (!dims || !out) return fail(JEPA_E_INVALID_ARG, "rope_table: null argument");
    TRY(check_dims(dims));
    rope_table(*dims, out);
    return JEPA_OK;
}

}  // extern "C"
