// Weight files: safetensors (bf16 models) and SLM2 (the same container holding Q8_0 block matrices and f32
// norms), mapped read-only and validated before any byte of weight data is used.
//
// Container ([P1] section 3 "File Layout and Safe Metadata Parsing"; [P2] "The safetensors format -- three
// regions"): an 8-byte little-endian header length N, N bytes of UTF-8 JSON mapping tensor names to
// {"dtype", "shape", "data_offsets": [begin, end]} (plus an optional "__metadata__" map of strings), then the
// data blob; offsets are relative to the blob.  Checks, each a typed error:
//   - N fits the file and the header is one well-formed JSON object (QW3_INVALID_MODEL otherwise);
//   - every entry has a known dtype, a shape of non-negative integers and end - begin == product(shape) times
//     the element size (34 bytes per 32 inputs for Q8_0) ([P2] parse_tensor_entry), in checked 64-bit
//     arithmetic (QW3_INTEGER_OVERFLOW);
//   - every end lies inside the blob (QW3_BOUNDS: [P1] "File Boundary Constraint");
//   - sorted by begin, the spans tile the blob exactly: no overlap and no hole (QW3_INVALID_MODEL: [P1]
//     "Monotonic Non-Overlapping Spans");
//   - every tensor starts at a file offset divisible by 8 (QW3_ALIGNMENT: [P1] "Strict Alignment");
//   - names are the Qwen3 inventory of [P2] ("expected_tensors"): model.embed_tokens.weight, model.norm.weight,
//     an optional tied lm_head.weight, and per layer the eleven block tensors; an unknown or duplicate name is
//     QW3_INVALID_MODEL.  Shapes and dtypes are then cross-checked against the configuration by the same code
//     that checks qw3_load_weights' tensors.
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P2] "M1 — Load the weights"
#include <fcntl.h>
#include <string.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "qw3.h"

namespace {

// ---- a strict JSON reader for the header (objects, arrays, strings, non-negative integers) ----------------
struct JVal {
    enum Kind { Null, Bool, Num, Str, Arr, Obj } kind = Null;
    bool neg = false, frac = false;  // a number with a sign or a fraction/exponent (never a valid offset)
    uint64_t num = 0;
    bool num_overflow = false;
    std::string str;
    std::vector<JVal> arr;
    std::vector<std::pair<std::string, JVal>> obj;
};

class JReader {
   public:
    JReader(const char *p, size_t n) : p_(p), e_(p + n) {}
    bool document(JVal &v) {
        ws();
        if (!value(v, 0)) return false;
        ws();
        return p_ == e_;
    }

   private:
    const char *p_, *e_;
    static constexpr int kMaxDepth = 16;
    void ws() {
        while (p_ < e_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
    }
    bool lit(const char *s) {
        const size_t n = strlen(s);
        if ((size_t)(e_ - p_) < n || memcmp(p_, s, n)) return false;
        p_ += n;
        return true;
    }
    static void put_utf8(std::string &o, uint32_t c) {
        if (c < 0x80) o += (char)c;
        else if (c < 0x800) o += (char)(0xC0 | (c >> 6)), o += (char)(0x80 | (c & 0x3F));
        else o += (char)(0xE0 | (c >> 12)), o += (char)(0x80 | ((c >> 6) & 0x3F)), o += (char)(0x80 | (c & 0x3F));
    }
    bool string(std::string &o) {
        if (p_ >= e_ || *p_ != '"') return false;
        ++p_;
        while (p_ < e_ && *p_ != '"') {
            const unsigned char c = (unsigned char)*p_++;
            if (c < 0x20) return false;  // control characters must be escaped
            if (c != '\\') {
                o += (char)c;
                continue;
            }
            if (p_ >= e_) return false;
            const char x = *p_++;
            switch (x) {
                case '"': o += '"'; break;
                case '\\': o += '\\'; break;
                case '/': o += '/'; break;
                case 'b': o += '\b'; break;
                case 'f': o += '\f'; break;
                case 'n': o += '\n'; break;
                case 'r': o += '\r'; break;
                case 't': o += '\t'; break;
                case 'u': {
                    if (e_ - p_ < 4) return false;
                    uint32_t c16 = 0;
                    for (int i = 0; i < 4; ++i) {
                        const char h = *p_++;
                        c16 <<= 4;
                        if (h >= '0' && h <= '9') c16 |= (uint32_t)(h - '0');
                        else if (h >= 'a' && h <= 'f') c16 |= (uint32_t)(h - 'a' + 10);
                        else if (h >= 'A' && h <= 'F') c16 |= (uint32_t)(h - 'A' + 10);
                        else return false;
                    }
                    if (c16 >= 0xD800 && c16 < 0xE000) return false;  // surrogates: no tensor name needs them
                    put_utf8(o, c16);
                    break;
                }
                default: return false;
            }
        }
        if (p_ >= e_) return false;
        ++p_;
        return true;
    }
    bool number(JVal &v) {
        v.kind = JVal::Num;
        if (*p_ == '-') {
            v.neg = true;
            ++p_;
        }
        if (p_ >= e_ || *p_ < '0' || *p_ > '9') return false;
        if (*p_ == '0' && p_ + 1 < e_ && p_[1] >= '0' && p_[1] <= '9') return false;  // no leading zeros
        while (p_ < e_ && *p_ >= '0' && *p_ <= '9') {
            const uint64_t d = (uint64_t)(*p_++ - '0');
            if (v.num > (UINT64_MAX - d) / 10) v.num_overflow = true;
            v.num = v.num * 10 + d;
        }
        if (p_ < e_ && (*p_ == '.' || *p_ == 'e' || *p_ == 'E')) {
            v.frac = true;
            if (*p_ == '.') {
                ++p_;
                if (p_ >= e_ || *p_ < '0' || *p_ > '9') return false;
                while (p_ < e_ && *p_ >= '0' && *p_ <= '9') ++p_;
            }
            if (p_ < e_ && (*p_ == 'e' || *p_ == 'E')) {
                ++p_;
                if (p_ < e_ && (*p_ == '+' || *p_ == '-')) ++p_;
                if (p_ >= e_ || *p_ < '0' || *p_ > '9') return false;
                while (p_ < e_ && *p_ >= '0' && *p_ <= '9') ++p_;
            }
        }
        return true;
    }
    bool value(JVal &v, int depth) {
        if (depth > kMaxDepth || p_ >= e_) return false;
        const char c = *p_;
        if (c == '{') {
            v.kind = JVal::Obj;
            ++p_;
            ws();
            if (p_ < e_ && *p_ == '}') {
                ++p_;
                return true;
            }
            for (;;) {
                ws();
                std::string k;
                if (!string(k)) return false;
                ws();
                if (p_ >= e_ || *p_ != ':') return false;
                ++p_;
                ws();
                v.obj.emplace_back(std::move(k), JVal());
                if (!value(v.obj.back().second, depth + 1)) return false;
                ws();
                if (p_ < e_ && *p_ == ',') {
                    ++p_;
                    continue;
                }
                if (p_ < e_ && *p_ == '}') {
                    ++p_;
                    return true;
                }
                return false;
            }
        }
        if (c == '[') {
            v.kind = JVal::Arr;
            ++p_;
            ws();
            if (p_ < e_ && *p_ == ']') {
                ++p_;
                return true;
            }
            for (;;) {
                ws();
                v.arr.emplace_back();
                if (!value(v.arr.back(), depth + 1)) return false;
                ws();
                if (p_ < e_ && *p_ == ',') {
                    ++p_;
                    continue;
                }
                if (p_ < e_ && *p_ == ']') {
                    ++p_;
                    return true;
                }
                return false;
            }
        }
        if (c == '"') {
            v.kind = JVal::Str;
            return string(v.str);
        }
        if (c == 't') return v.kind = JVal::Bool, lit("true");
        if (c == 'f') return v.kind = JVal::Bool, lit("false");
        if (c == 'n') return v.kind = JVal::Null, lit("null");
        return number(v);
    }
};

// ---- checked arithmetic ----------------------------------------------------------------------------------
bool mul_ok(uint64_t a, uint64_t b, uint64_t &r) {
    if (a && b > UINT64_MAX / a) return false;
    r = a * b;
    return true;
}

// ---- the tensor directory ----------------------------------------------------------------------------------
struct Entry {
    std::string name;
    int32_t kind = -1, layer = -1, dtype = 0;
    std::vector<uint64_t> shape;
    uint64_t begin = 0, end = 0;
};

// Inventory name -> (kind, layer) ([P2] expected_tensors: 3 global tensors + 11 per block).
bool classify(const std::string &name, int32_t &kind, int32_t &layer) {
    layer = -1;
    if (name == "model.embed_tokens.weight") return kind = QW3_T_EMBED, true;
    if (name == "model.norm.weight") return kind = QW3_T_FINAL_NORM, true;
    if (name == "lm_head.weight") return kind = QW3_T_LM_HEAD, true;
    static const char *kPre = "model.layers.";
    if (name.compare(0, strlen(kPre), kPre)) return false;
    size_t i = strlen(kPre);
    if (i >= name.size() || name[i] < '0' || name[i] > '9' || (name[i] == '0' && i + 1 < name.size() && name[i + 1] != '.'))
        return false;
    uint64_t l = 0;
    while (i < name.size() && name[i] >= '0' && name[i] <= '9') {
        l = l * 10 + (uint64_t)(name[i++] - '0');
        if (l > (1u << 20)) return false;
    }
    if (i >= name.size() || name[i] != '.') return false;
    const std::string rest = name.substr(i + 1);
    static const std::pair<const char *, int32_t> kSlots[] = {
        {"input_layernorm.weight", QW3_T_ATTN_NORM}, {"self_attn.q_proj.weight", QW3_T_Q},
        {"self_attn.k_proj.weight", QW3_T_K},        {"self_attn.v_proj.weight", QW3_T_V},
        {"self_attn.q_norm.weight", QW3_T_Q_NORM},   {"self_attn.k_norm.weight", QW3_T_K_NORM},
        {"self_attn.o_proj.weight", QW3_T_O},        {"post_attention_layernorm.weight", QW3_T_MLP_NORM},
        {"mlp.gate_proj.weight", QW3_T_GATE},        {"mlp.up_proj.weight", QW3_T_UP},
        {"mlp.down_proj.weight", QW3_T_DOWN}};
    for (const auto &s : kSlots)
        if (rest == s.first) {
            kind = s.second;
            layer = (int32_t)l;
            return true;
        }
    return false;
}

// dtype name -> (qw3 dtype, bytes per element; Q8_0 handled separately)
bool dtype_of(const std::string &s, int32_t &dt, uint64_t &eb) {
    if (s == "BF16") return dt = QW3_DT_BF16, eb = 2, true;
    if (s == "F32") return dt = QW3_DT_F32, eb = 4, true;
    if (s == "Q8_0") return dt = QW3_DT_Q8_0, eb = 0, true;
    return false;
}

struct Mapped {
    void *base = MAP_FAILED;
    size_t size = 0;
    ~Mapped() {
        if (base != MAP_FAILED) (void)munmap(base, size);
    }
};

// Maps `path` and validates its header; fills the entries (in header order) and the blob's file offset.
int32_t parse_file(const char *path, Mapped &mp, std::vector<Entry> &ents, uint64_t &blob_off) {
    if (!path) return QW3_INVALID_ARGUMENT;
    const int fd = open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return QW3_INVALID_ARGUMENT;
    struct stat stt;
    if (fstat(fd, &stt) != 0 || !S_ISREG(stt.st_mode) || stt.st_size < 8) {
        close(fd);
        return QW3_INVALID_MODEL;
    }
    mp.size = (size_t)stt.st_size;
    mp.base = mmap(nullptr, mp.size, PROT_READ, MAP_PRIVATE, fd, 0);
    close(fd);
    if (mp.base == MAP_FAILED) return QW3_INVALID_ARGUMENT;
    const uint8_t *b = (const uint8_t *)mp.base;
    uint64_t n = 0;
    for (int i = 7; i >= 0; --i) n = (n << 8) | b[i];  // little-endian u64
    if (n > mp.size - 8) return QW3_BOUNDS;
    JVal root;
    if (!JReader((const char *)b + 8, (size_t)n).document(root) || root.kind != JVal::Obj) return QW3_INVALID_MODEL;
    blob_off = 8 + n;
    const uint64_t blob = mp.size - blob_off;
    std::map<std::string, int> names;
    for (const auto &kv : root.obj) {
        if (!names.emplace(kv.first, 1).second) return QW3_INVALID_MODEL;  // duplicate key
        if (kv.first == "__metadata__") {
            if (kv.second.kind != JVal::Obj) return QW3_INVALID_MODEL;
            for (const auto &m : kv.second.obj)
                if (m.second.kind != JVal::Str) return QW3_INVALID_MODEL;
            continue;
        }
        const JVal &t = kv.second;
        if (t.kind != JVal::Obj) return QW3_INVALID_MODEL;
        const JVal *dt = nullptr, *sh = nullptr, *off = nullptr;
        for (const auto &f : t.obj) {
            if (f.first == "dtype") dt = &f.second;
            else if (f.first == "shape") sh = &f.second;
            else if (f.first == "data_offsets") off = &f.second;
            else return QW3_INVALID_MODEL;
        }
        if (!dt || !sh || !off || dt->kind != JVal::Str || sh->kind != JVal::Arr || off->kind != JVal::Arr ||
            off->arr.size() != 2)
            return QW3_INVALID_MODEL;
        Entry e;
        e.name = kv.first;
        if (!classify(e.name, e.kind, e.layer)) return QW3_INVALID_MODEL;
        uint64_t eb = 0;
        if (!dtype_of(dt->str, e.dtype, eb)) return QW3_INVALID_MODEL;
        for (const JVal &d : sh->arr) {
            if (d.kind != JVal::Num || d.neg || d.frac) return QW3_INVALID_MODEL;
            if (d.num_overflow) return QW3_INTEGER_OVERFLOW;
            e.shape.push_back(d.num);
        }
        for (int i = 0; i < 2; ++i) {
            const JVal &o = off->arr[i];
            if (o.kind != JVal::Num || o.neg || o.frac) return QW3_INVALID_MODEL;
            if (o.num_overflow) return QW3_INTEGER_OVERFLOW;
        }
        e.begin = off->arr[0].num;
        e.end = off->arr[1].num;
        if (e.end < e.begin) return QW3_INVALID_MODEL;
        if (e.end > blob) return QW3_BOUNDS;
        // byte size implied by the shape ([P2] parse_tensor_entry: end - start == shape * dtype size)
        uint64_t bytes = 0;
        if (e.dtype == QW3_DT_Q8_0) {
            if (e.shape.size() != 2 || e.shape[1] % 32) return QW3_INVALID_MODEL;  // whole blocks only
            if (!mul_ok(e.shape[0], e.shape[1] / 32, bytes) || !mul_ok(bytes, 34, bytes)) return QW3_INTEGER_OVERFLOW;
        } else {
            bytes = eb;
            for (uint64_t d : e.shape)
                if (!mul_ok(bytes, d, bytes)) return QW3_INTEGER_OVERFLOW;
        }
        if (e.end - e.begin != bytes) return QW3_INVALID_MODEL;
        if ((blob_off + e.begin) % 8) return QW3_ALIGNMENT;
        ents.push_back(std::move(e));
    }
    // the spans tile the blob: sorted by start, each begins where the previous ended
    std::vector<const Entry *> by(ents.size());
    for (size_t i = 0; i < ents.size(); ++i) by[i] = &ents[i];
    std::sort(by.begin(), by.end(), [](const Entry *x, const Entry *y) { return x->begin < y->begin; });
    uint64_t at = 0;
    for (const Entry *e : by) {
        if (e->begin != at) return QW3_INVALID_MODEL;  // overlap (begin < at) or hole (begin > at)
        at = e->end;
    }
    if (at != blob) return QW3_INVALID_MODEL;  // trailing bytes nobody owns
    return QW3_OK;
}

// Canonical tensor list ([rows, cols]; vectors as [1, n]) pointing into the mapping.
int32_t to_tensors(const std::vector<Entry> &ents, const uint8_t *blob, std::vector<qw3_tensor_t> &out) {
    for (const Entry &e : ents) {
        qw3_tensor_t t{};
        t.kind = e.kind;
        t.layer = e.layer;
        t.dtype = e.dtype;
        if (e.shape.size() == 1) {
            t.rows = 1;
            t.cols = (int64_t)e.shape[0];
        } else if (e.shape.size() == 2) {
            t.rows = (int64_t)e.shape[0];
            t.cols = (int64_t)e.shape[1];
        } else {
            return QW3_INVALID_MODEL;
        }
        if (t.rows < 0 || t.cols < 0) return QW3_INTEGER_OVERFLOW;
        t.data = blob + e.begin;
        t.scales = nullptr;
        out.push_back(t);
    }
    return QW3_OK;
}

}  // namespace

extern "C" {

int32_t qw3_inspect_file(const char *path, qw3_file_report_t *out) {
    if (!out) return QW3_INVALID_ARGUMENT;
    memset(out, 0, sizeof(*out));
    Mapped mp;
    std::vector<Entry> ents;
    uint64_t blob_off = 0;
    const int32_t rc = parse_file(path, mp, ents, blob_off);
    if (rc != QW3_OK) return rc;
    int64_t stored = 0, lm = 0, embed = 0;
    int32_t max_layer = -1;
    for (const Entry &e : ents) {
        int64_t n = 1;
        for (uint64_t d : e.shape) n *= (int64_t)d;
        stored += n;
        if (e.kind == QW3_T_LM_HEAD) lm = n;
        if (e.kind == QW3_T_EMBED) embed = n;
        max_layer = std::max(max_layer, e.layer);
    }
    out->n_tensors = (int64_t)ents.size();
    out->stored_params = stored;
    out->logical_params = stored - lm;  // a tied lm_head is a redundant copy ([P2] "Tied != absent")
    out->embed_params = embed;
    out->n_layers = max_layer + 1;
    out->lm_head_present = lm ? 1 : 0;
    out->header_bytes = (int64_t)blob_off - 8;
    return QW3_OK;
}

int32_t qw3_load_file(uint64_t handle, const char *path, void *stream) {
    Mapped mp;
    std::vector<Entry> ents;
    uint64_t blob_off = 0;
    int32_t rc = parse_file(path, mp, ents, blob_off);
    if (rc != QW3_OK) return rc;
    std::vector<qw3_tensor_t> ts;
    rc = to_tensors(ents, (const uint8_t *)mp.base + blob_off, ts);
    if (rc != QW3_OK) return rc;
    // shapes, dtypes, completeness and the tied lm_head are checked against the configuration here; the call
    // returns after its copies completed, so the mapping may be released afterwards
    return qw3_load_weights(handle, ts.data(), (int32_t)ts.size(), stream);
}

}  // extern "C"
