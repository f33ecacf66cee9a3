// GGUF model files: the container read on the host, its jepa.* keys turned
// into jepa_dims and its tensors handed to jepa_create straight from a
// read-only mapping of the file.
//
// Container (GGUF versions 2 and 3, little-endian): "GGUF", u32 version,
// u64 tensor count, u64 key count; the keys (string name, u32 value type,
// value); the tensor records (string name, u32 dimension count, u64 per
// dimension with the row length first, u32 ggml type, u64 offset into the
// data section); the data section at the next multiple of general.alignment
// (32 when absent).  A string is a u64 byte count and the bytes.
// Every read is checked against the end of the file; nothing is trusted.
#include <errno.h>
#include <math.h>
#include <fcntl.h>
#include <stdint.h>
#include <string.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <map>
#include <string>
#include <vector>

#include "host.hpp"

using jepa::fail;

namespace {

// GGUF value types
enum : uint32_t {
    GV_U8 = 0, GV_I8 = 1, GV_U16 = 2, GV_I16 = 3, GV_U32 = 4, GV_I32 = 5, GV_F32 = 6, GV_BOOL = 7,
    GV_STR = 8, GV_ARR = 9, GV_U64 = 10, GV_I64 = 11, GV_F64 = 12
};

// ggml tensor types: (name, weights per block, bytes per block, jepa dtype
// or -1 when this library does not run it)
struct GgmlType { uint32_t id; const char *name; int64_t per, bytes; int dt; };
constexpr GgmlType kTypes[] = {
    {0, "f32", 1, 4, JEPA_F32},     {1, "f16", 1, 2, JEPA_F16},     {2, "q4_0", 32, 18, JEPA_Q4_0},
    {3, "q4_1", 32, 20, -1},        {6, "q5_0", 32, 22, -1},        {7, "q5_1", 32, 24, -1},
    {8, "q8_0", 32, 34, JEPA_Q8_0}, {12, "q4_K", 256, 144, JEPA_Q4_K}, {13, "q5_K", 256, 176, -1},
    {14, "q6_K", 256, 210, JEPA_Q6_K}, {30, "bf16", 1, 2, JEPA_BF16},
};

const GgmlType *ggml_type(uint32_t id) {
    for (const auto &t : kTypes)
        if (t.id == id) return &t;
    return nullptr;
}

// a name from the file as it may appear in a message: printable ASCII,
// at most 96 characters
std::string shown(const std::string &s) {
    std::string o;
    for (size_t i = 0; i < s.size() && o.size() < 96; ++i) o += (s[i] >= 32 && s[i] < 127) ? s[i] : '?';
    return o;
}

constexpr uint64_t MAX_STRING = 1u << 20;      // longer key / tensor names are refused
constexpr uint64_t MAX_COUNT = 1u << 24;       // tensors, keys, array elements
constexpr int MAX_DIMS = 4;

struct Value {
    uint32_t type = 0;
    bool is_num = false;
    double num = 0;                 // numeric scalars (and bools)
    int64_t inum = 0;
    std::string str;
    uint32_t arr_type = 0;
    uint64_t arr_n = 0;
    std::vector<double> arr;        // numeric array elements
};

struct TensorRec {
    std::string name;
    int64_t ne[MAX_DIMS] = {1, 1, 1, 1};
    int n_dims = 0;
    const GgmlType *type = nullptr;
    uint64_t offset = 0;
    uint64_t bytes = 0;
};

struct Parsed {
    uint32_t version = 0;
    std::map<std::string, Value> kv;
    std::vector<TensorRec> tensors;
    uint64_t alignment = 32, data_offset = 0;
};

class Reader {
  public:
    Reader(const uint8_t *p, size_t n) : p_(p), n_(n) {}
    size_t pos() const { return pos_; }
    size_t remaining() const { return n_ - pos_; }
    template <typename T> bool get(T &v) {
        if (n_ - pos_ < sizeof(T)) return false;
        memcpy(&v, p_ + pos_, sizeof(T));
        pos_ += sizeof(T);
        return true;
    }
    bool str(std::string &s) {
        uint64_t len;
        if (!get(len) || len > MAX_STRING || len > n_ - pos_) return false;
        s.assign((const char *)p_ + pos_, (size_t)len);
        pos_ += (size_t)len;
        return true;
    }

  private:
    const uint8_t *p_;
    size_t n_, pos_ = 0;
};

size_t scalar_bytes(uint32_t t) {
    switch (t) {
        case GV_U8: case GV_I8: case GV_BOOL: return 1;
        case GV_U16: case GV_I16: return 2;
        case GV_U32: case GV_I32: case GV_F32: return 4;
        case GV_U64: case GV_I64: case GV_F64: return 8;
    }
    return 0;
}

// a float as an integer where one is wanted (0 outside int64's range)
int64_t float_to_int(double v) { return (v > -9.2e18 && v < 9.2e18) ? (int64_t)v : 0; }

// a numeric scalar of type t at the reader, as double and int64
bool read_number(Reader &r, uint32_t t, double &d, int64_t &i) {
    switch (t) {
        case GV_U8: { uint8_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_I8: { int8_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_BOOL: { uint8_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_U16: { uint16_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_I16: { int16_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_U32: { uint32_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_I32: { int32_t v; if (!r.get(v)) return false; d = v; i = v; return true; }
        case GV_F32: { float v; if (!r.get(v)) return false; d = v; i = float_to_int(v); return true; }
        case GV_U64: { uint64_t v; if (!r.get(v)) return false; d = (double)v; i = (int64_t)v; return true; }
        case GV_I64: { int64_t v; if (!r.get(v)) return false; d = (double)v; i = v; return true; }
        case GV_F64: { double v; if (!r.get(v)) return false; d = v; i = float_to_int(v); return true; }
    }
    return false;
}

jepa_status parse(const uint8_t *p, size_t n, Parsed &out) {
    Reader r(p, n);
    char magic[4];
    if (!r.get(magic) || memcmp(magic, "GGUF", 4))
        return fail(JEPA_E_FORMAT, "gguf: not a GGUF file (bad magic)");
    uint32_t version;
    uint64_t n_tensors, n_kv;
    if (!r.get(version)) return fail(JEPA_E_FORMAT, "gguf: truncated header");
    if (version != 2 && version != 3)
        return fail(JEPA_E_UNSUPPORTED, "gguf: version %u (2 and 3 are read)", version);
    if (!r.get(n_tensors) || !r.get(n_kv)) return fail(JEPA_E_FORMAT, "gguf: truncated header");
    if (n_tensors > MAX_COUNT || n_kv > MAX_COUNT)
        return fail(JEPA_E_FORMAT, "gguf: %llu tensors / %llu keys is implausible", (unsigned long long)n_tensors,
                    (unsigned long long)n_kv);
    out.version = version;
    for (uint64_t k = 0; k < n_kv; ++k) {
        std::string key;
        Value v;
        if (!r.str(key) || !r.get(v.type)) return fail(JEPA_E_FORMAT, "gguf: truncated key %llu", (unsigned long long)k);
        if (v.type == GV_STR) {
            if (!r.str(v.str)) return fail(JEPA_E_FORMAT, "gguf: truncated string value of '%s'", shown(key).c_str());
        } else if (v.type == GV_ARR) {
            if (!r.get(v.arr_type) || !r.get(v.arr_n))
                return fail(JEPA_E_FORMAT, "gguf: truncated array header of '%s'", shown(key).c_str());
            if (v.arr_n > MAX_COUNT) return fail(JEPA_E_FORMAT, "gguf: array '%s' too long", shown(key).c_str());
            if (v.arr_type == GV_STR) {
                for (uint64_t e = 0; e < v.arr_n; ++e) {
                    std::string s;
                    if (!r.str(s)) return fail(JEPA_E_FORMAT, "gguf: truncated string array '%s'", shown(key).c_str());
                }
            } else if (scalar_bytes(v.arr_type)) {
                if (v.arr_n > r.remaining() / scalar_bytes(v.arr_type))
                    return fail(JEPA_E_FORMAT, "gguf: truncated array '%s'", shown(key).c_str());
                v.arr.resize((size_t)v.arr_n);
                for (uint64_t e = 0; e < v.arr_n; ++e) {
                    int64_t i;
                    if (!read_number(r, v.arr_type, v.arr[(size_t)e], i))
                        return fail(JEPA_E_FORMAT, "gguf: truncated array '%s'", shown(key).c_str());
                }
            } else {
                return fail(JEPA_E_FORMAT, "gguf: array '%s' has element type %u", shown(key).c_str(), v.arr_type);
            }
        } else if (scalar_bytes(v.type)) {
            if (!read_number(r, v.type, v.num, v.inum))
                return fail(JEPA_E_FORMAT, "gguf: truncated value of '%s'", shown(key).c_str());
            v.is_num = true;
        } else {
            return fail(JEPA_E_FORMAT, "gguf: key '%s' has value type %u", shown(key).c_str(), v.type);
        }
        if (out.kv.count(key)) return fail(JEPA_E_FORMAT, "gguf: key '%s' given twice", shown(key).c_str());
        out.kv[key] = std::move(v);
    }
    auto al = out.kv.find("general.alignment");
    if (al != out.kv.end()) {
        if (!al->second.is_num || al->second.inum < 8 || al->second.inum > (1 << 20) || al->second.inum % 8)
            return fail(JEPA_E_FORMAT, "gguf: general.alignment must be a multiple of 8 up to 2^20");
        out.alignment = (uint64_t)al->second.inum;
    }
    out.tensors.resize((size_t)n_tensors);
    for (uint64_t t = 0; t < n_tensors; ++t) {
        TensorRec &tr = out.tensors[(size_t)t];
        uint32_t nd, type;
        if (!r.str(tr.name) || !r.get(nd)) return fail(JEPA_E_FORMAT, "gguf: truncated tensor record %llu", (unsigned long long)t);
        if (nd < 1 || nd > MAX_DIMS)
            return fail(JEPA_E_FORMAT, "gguf: tensor '%s' has %u dimensions", shown(tr.name).c_str(), nd);
        tr.n_dims = (int)nd;
        uint64_t elems = 1;
        for (uint32_t i = 0; i < nd; ++i) {
            uint64_t ne;
            if (!r.get(ne)) return fail(JEPA_E_FORMAT, "gguf: truncated tensor record '%s'", shown(tr.name).c_str());
            if (ne == 0 || ne > (1ull << 40) || elems > (1ull << 40) / ne)
                return fail(JEPA_E_FORMAT, "gguf: tensor '%s' has a bad dimension", shown(tr.name).c_str());
            tr.ne[i] = (int64_t)ne;
            elems *= ne;
        }
        if (!r.get(type) || !r.get(tr.offset))
            return fail(JEPA_E_FORMAT, "gguf: truncated tensor record '%s'", shown(tr.name).c_str());
        tr.type = ggml_type(type);
        if (!tr.type) return fail(JEPA_E_UNSUPPORTED, "gguf: tensor '%s' has ggml type %u", shown(tr.name).c_str(), type);
        if (tr.ne[0] % tr.type->per)
            return fail(JEPA_E_FORMAT, "gguf: tensor '%s' row length %lld is not a whole number of %s blocks",
                        shown(tr.name).c_str(), (long long)tr.ne[0], tr.type->name);
        tr.bytes = elems / (uint64_t)tr.type->per * (uint64_t)tr.type->bytes;
        if (tr.offset % out.alignment)
            return fail(JEPA_E_FORMAT, "gguf: tensor '%s' offset %llu is not aligned to %llu", shown(tr.name).c_str(),
                        (unsigned long long)tr.offset, (unsigned long long)out.alignment);
    }
    const uint64_t data = (r.pos() + out.alignment - 1) / out.alignment * out.alignment;
    if (data > n) return fail(JEPA_E_FORMAT, "gguf: file ends before its data section");
    out.data_offset = data;
    for (const TensorRec &tr : out.tensors)
        if (tr.offset > n - data || tr.bytes > n - data - tr.offset)
            return fail(JEPA_E_FORMAT, "gguf: tensor '%s' (%llu bytes at %llu) runs past the end of the file",
                        shown(tr.name).c_str(), (unsigned long long)tr.bytes, (unsigned long long)tr.offset);
    return JEPA_OK;
}

// ---- the jepa.* keys -> jepa_dims ------------------------------------------
jepa_status int_key(const Parsed &P, const char *key, bool required, int64_t dflt, int32_t &out) {
    auto it = P.kv.find(key);
    if (it == P.kv.end()) {
        if (required) return fail(JEPA_E_FORMAT, "gguf: key '%s' is missing", key);
        out = (int32_t)dflt;
        return JEPA_OK;
    }
    const Value &v = it->second;
    if (!v.is_num || v.type == GV_F32 || v.type == GV_F64 || v.inum < 0 || v.inum > INT32_MAX)
        return fail(JEPA_E_FORMAT, "gguf: key '%s' must be a non-negative integer", key);
    out = (int32_t)v.inum;
    return JEPA_OK;
}

jepa_status vec3_key(const Parsed &P, const char *key, float out[3]) {
    auto it = P.kv.find(key);
    if (it == P.kv.end()) return fail(JEPA_E_FORMAT, "gguf: key '%s' is missing", key);
    const Value &v = it->second;
    if (v.type != GV_ARR || v.arr.size() != 3 || (v.arr_type != GV_F32 && v.arr_type != GV_F64))
        return fail(JEPA_E_FORMAT, "gguf: key '%s' must be an array of 3 floats", key);
    for (int c = 0; c < 3; ++c) {
        if (!(fabs(v.arr[c]) < 1e30)) return fail(JEPA_E_FORMAT, "gguf: key '%s' holds a non-finite value", key);
        out[c] = (float)v.arr[c];
    }
    return JEPA_OK;
}

#define TRY_G(expr)                           \
    do {                                      \
        jepa_status st_ = (expr);             \
        if (st_ != JEPA_OK) return st_;       \
    } while (0)

jepa_status dims_of(const Parsed &P, jepa_dims &d) {
    memset(&d, 0, sizeof d);
    auto arch = P.kv.find("general.architecture");
    if (arch == P.kv.end() || arch->second.type != GV_STR)
        return fail(JEPA_E_FORMAT, "gguf: general.architecture is missing");
    if (arch->second.str != "jepa")
        return fail(JEPA_E_UNSUPPORTED, "gguf: architecture '%s' (this library reads 'jepa')", shown(arch->second.str).c_str());
    TRY_G(int_key(P, "jepa.dim", true, 0, d.dim));
    TRY_G(int_key(P, "jepa.depth", true, 0, d.depth));
    TRY_G(int_key(P, "jepa.heads", true, 0, d.heads));
    TRY_G(int_key(P, "jepa.mlp_dim", true, 0, d.mlp_dim));
    TRY_G(int_key(P, "jepa.patch", true, 0, d.patch));
    TRY_G(int_key(P, "jepa.tubelet", false, 1, d.tubelet));
    TRY_G(int_key(P, "jepa.img_h", true, 0, d.img_h));
    TRY_G(int_key(P, "jepa.img_w", true, 0, d.img_w));
    TRY_G(int_key(P, "jepa.frames", false, 1, d.frames));
    TRY_G(int_key(P, "jepa.has_cls", true, 0, d.has_cls));
    TRY_G(int_key(P, "jepa.rope", false, 0, d.rope));
    TRY_G(int_key(P, "jepa.head.blocks", false, 0, d.head_blocks));
    TRY_G(int_key(P, "jepa.head.classes", false, 0, d.head_classes));
    d.mask = JEPA_MASK_BIDIR;
    auto m = P.kv.find("jepa.mask");
    if (m != P.kv.end()) {
        if (m->second.type != GV_STR) return fail(JEPA_E_FORMAT, "gguf: jepa.mask must be a string");
        if (m->second.str == "block_causal") d.mask = JEPA_MASK_BLOCK_CAUSAL;
        else if (m->second.str != "bidirectional")
            return fail(JEPA_E_FORMAT, "gguf: jepa.mask '%s' (bidirectional or block_causal)", shown(m->second.str).c_str());
    }
    d.ln_eps = 1e-6f;
    auto e = P.kv.find("jepa.ln_eps");
    if (e != P.kv.end()) {
        if (!e->second.is_num || !(e->second.num > 0 && e->second.num < 1))
            return fail(JEPA_E_FORMAT, "gguf: jepa.ln_eps must be a number in (0, 1)");
        d.ln_eps = (float)e->second.num;
    }
    TRY_G(vec3_key(P, "jepa.pre.mean", d.mean));
    TRY_G(vec3_key(P, "jepa.pre.std", d.std));
    d.act_dtype = JEPA_F32;
    return JEPA_OK;
}

// A read-only mapping of a whole file, unmapped on scope exit.
struct Mapping {
    const uint8_t *p = nullptr;
    size_t n = 0;
    ~Mapping() {
        if (p) munmap((void *)p, n);
    }
    jepa_status open(const char *path) {
        const int fd = ::open(path, O_RDONLY | O_CLOEXEC);
        if (fd < 0) return fail(JEPA_E_INVALID_ARG, "gguf: cannot open '%s': %s", path, strerror(errno));
        struct stat st;
        if (fstat(fd, &st) != 0 || !S_ISREG(st.st_mode)) {
            ::close(fd);
            return fail(JEPA_E_INVALID_ARG, "gguf: '%s' is not a regular file", path);
        }
        n = (size_t)st.st_size;
        if (n == 0) {
            ::close(fd);
            return fail(JEPA_E_FORMAT, "gguf: '%s' is empty", path);
        }
        void *m = mmap(nullptr, n, PROT_READ, MAP_PRIVATE, fd, 0);
        ::close(fd);
        if (m == MAP_FAILED) return fail(JEPA_E_INVALID_ARG, "gguf: cannot map '%s': %s", path, strerror(errno));
        p = (const uint8_t *)m;
        return JEPA_OK;
    }
};

}  // namespace

extern "C" {

const char *jepa_file_type_name(int code) {
    // general.file_type codes (jepa.cpp Quantization page, "The rule")
    switch (code) {
        case 0: return "f32";
        case 1: return "f16";
        case 2: return "q4_0";
        case 3: return "q4_1";
        case 7: return "q8_0";
        case 8: return "q5_0";
        case 9: return "q5_1";
        case 12: return "q4_k";
        case 13: return "q5_k";
        case 14: return "q6_k";
    }
    return nullptr;
}

jepa_status jepa_gguf_read_info(const char *path, jepa_gguf_info *info) {
    if (!path || !info) return fail(JEPA_E_INVALID_ARG, "gguf: null argument");
    memset(info, 0, sizeof *info);
    Mapping map;
    TRY_G(map.open(path));
    Parsed P;
    TRY_G(parse(map.p, map.n, P));
    TRY_G(dims_of(P, info->dims));
    info->version = (int32_t)P.version;
    info->file_type = -1;
    auto ft = P.kv.find("general.file_type");
    if (ft != P.kv.end()) {
        if (!ft->second.is_num || ft->second.inum < 0 || ft->second.inum > INT32_MAX)
            return fail(JEPA_E_FORMAT, "gguf: general.file_type must be a non-negative integer");
        info->file_type = (int32_t)ft->second.inum;
    }
    info->n_tensors = (int64_t)P.tensors.size();
    info->n_kv = (int64_t)P.kv.size();
    info->alignment = (int64_t)P.alignment;
    info->data_offset = (int64_t)P.data_offset;
    for (const TensorRec &t : P.tensors) info->tensor_bytes += (int64_t)t.bytes;
    return JEPA_OK;
}

jepa_status jepa_create_from_gguf(const char *path, int act_dtype, jepa_ctx **out) {
    if (!path || !out) return fail(JEPA_E_INVALID_ARG, "gguf: null argument");
    *out = nullptr;
    Mapping map;
    TRY_G(map.open(path));
    Parsed P;
    TRY_G(parse(map.p, map.n, P));
    jepa_dims d;
    TRY_G(dims_of(P, d));
    std::vector<jepa_tensor> ts(P.tensors.size());
    bool any_f16 = false, any_bf16 = false, all_f32 = true;
    for (size_t i = 0; i < P.tensors.size(); ++i) {
        const TensorRec &tr = P.tensors[i];
        if (tr.type->dt < 0)
            return fail(JEPA_E_UNSUPPORTED, "gguf: tensor '%s' is %s, which this library does not run", shown(tr.name).c_str(),
                        tr.type->name);
        int64_t ne1 = 1;
        for (int k = 1; k < tr.n_dims; ++k) ne1 *= tr.ne[k];
        ts[i] = jepa_tensor{tr.name.c_str(), tr.type->dt, tr.ne[0], ne1, map.p + P.data_offset + tr.offset,
                            (size_t)tr.bytes};
        all_f32 &= tr.type->dt == JEPA_F32;
        any_bf16 |= tr.type->dt == JEPA_BF16;
        any_f16 |= tr.type->dt != JEPA_F32 && tr.type->dt != JEPA_BF16;
    }
    if (act_dtype < 0) act_dtype = all_f32 ? JEPA_F32 : (any_bf16 && !any_f16) ? JEPA_BF16 : JEPA_F16;
    d.act_dtype = act_dtype;
    return jepa_create(&d, ts.data(), (int)ts.size(), out);
}

}  // extern "C"
