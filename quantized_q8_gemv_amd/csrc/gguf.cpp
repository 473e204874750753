// gguf.cpp -- GGUF model-file reader (host side): header, metadata, tensor
// directory, and tensor bytes by name.
//
// The pages describe the step before the forward ("生成一个 token", section
// "读 GGUF：130 ms，只读头部"): reading the magic, the version, the metadata
// key/values and the tensor directory, recording where the tensor data starts
// and reading no weights; then ("建模型：按名字取张量") seeking to each named
// tensor's offset in the data region and reading its raw bytes. The model's
// hyper-parameters come from llama.* keys, a missing one failing with "cannot
// find {key} in metadata" ("量化 llama 的一次前向", section "from_gguf：键名写死了
// llama."), and general.architecture selects the rope pairing (section "RoPE：两
// 种约定，按架构名选"). The byte format itself is not on the pages; it follows
// the public GGUF specification (version 2 and 3): little-endian; magic
// "GGUF"; u32 version; u64 tensor count; u64 metadata count; each metadata
// entry = string key, u32 value type, value; each tensor entry = string name,
// u32 dimension count, u64 dimensions (innermost first), u32 tensor type, u64
// offset into the data region; the data region starts at the next multiple of
// general.alignment (32 when absent). Strings are a u64 length and bytes.
//
// The reader never trusts a length: every count and size is checked against
// the file size before it is used, so a truncated or corrupt file yields
// Q8L_E_FORMAT instead of a large allocation or an out-of-range read.

#include <cstdio>
#include <sys/types.h>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/q8l.h"

namespace {

enum GgufType : uint32_t {
    G_U8 = 0, G_I8 = 1, G_U16 = 2, G_I16 = 3, G_U32 = 4, G_I32 = 5, G_F32 = 6, G_BOOL = 7,
    G_STRING = 8, G_ARRAY = 9, G_U64 = 10, G_I64 = 11, G_F64 = 12
};

// Tensor element types of the file format this library can bind. Q4_0 and
// Q5_0 blocks hold d * (an integer in [-8, 7] or [-16, 15]) per 32 weights:
// the same values as a Q8_0 block with the same d, so they are read as Q8_0
// (converted exactly while reading). Q4_K and Q6_K (256-weight blocks of 144
// and 210 bytes) are read as they are.
constexpr uint32_t kTypeF32 = 0;
constexpr uint32_t kTypeQ4_0 = 2;
constexpr uint32_t kTypeQ5_0 = 6;
constexpr uint32_t kTypeQ8_0 = 8;
constexpr uint32_t kTypeQ4_K = 12;
constexpr uint32_t kTypeQ6_K = 14;

struct Value {
    uint32_t type = 0;
    // scalars (integers widened, floats as double); strings; arrays keep
    // their element type and count only
    bool is_int = false, is_float = false;
    int64_t i = 0;
    uint64_t u = 0;
    double f = 0.0;
    std::string s;
    uint32_t arr_type = 0;
    uint64_t arr_count = 0;
};

struct TensorInfo {
    std::string name;
    std::vector<uint64_t> dims;
    uint32_t type = 0;
    uint64_t offset = 0;      // within the data region
    uint64_t file_bytes = 0;  // bytes in the file
    uint64_t nbytes = 0;      // bytes as read (Q8_0 for the 32-weight integer formats), 0 if unreadable
    bool native = false;      // Q5_0 read as it is (see q5_native_role)
};

bool q8_family(uint32_t t) { return t == kTypeQ4_0 || t == kTypeQ5_0 || t == kTypeQ8_0; }
bool k_family(uint32_t t) { return t == kTypeQ4_K || t == kTypeQ6_K; }

uint64_t block_bytes(uint32_t t) { return t == kTypeQ4_0 ? 18 : t == kTypeQ5_0 ? 22 : 34; }

// Q5_0 tensors that the model binds in their own format: the seven
// projections of a layer ("blk.<n>.<role>.weight") with rows of at least
// kQ5NativeMinCols weights. Others (the embedding, the output matrix, and
// shorter rows) are read as Q8_0: rows under 2048 weights take the
// latency-bound wave-per-row decode kernels, where unpacking the fifth bits
// costs more than the bytes it saves (135M shape, every projection Q5_0:
// 567 us/token streamed as Q5_0 against 469 as Q8_0; the 7B-class shape,
// rows of 4096: 2000 against 2206).
constexpr uint64_t kQ5NativeMinCols = 2048;

bool q5_native_role(const std::string &name) {
    if (name.compare(0, 4, "blk.") != 0) return false;
    size_t p = 4;
    while (p < name.size() && name[p] >= '0' && name[p] <= '9') ++p;
    if (p == 4 || p >= name.size() || name[p] != '.') return false;
    const std::string role = name.substr(p + 1);
    for (const char *r : {"attn_q.weight", "attn_k.weight", "attn_v.weight", "attn_output.weight",
                          "ffn_gate.weight", "ffn_up.weight", "ffn_down.weight"})
        if (role == r) return true;
    return false;
}

// One Q4_0 / Q5_0 block (file layout: public GGUF block definitions) as a
// Q8_0 block: the f16 scale is copied, weight i of the block becomes the int8
// (nibble - 8), resp. ((nibble | fifth bit << 4) - 16); nibble i < 16 is the
// low half of byte i, nibble i + 16 its high half.
void to_q8_0(uint32_t type, const uint8_t *src, uint8_t *dst) {
    dst[0] = src[0];
    dst[1] = src[1];
    int8_t *q = reinterpret_cast<int8_t *>(dst + 2);
    if (type == kTypeQ4_0) {
        for (int i = 0; i < 16; ++i) {
            q[i] = int8_t((src[2 + i] & 0x0f) - 8);
            q[i + 16] = int8_t((src[2 + i] >> 4) - 8);
        }
        return;
    }
    uint32_t qh = 0;
    std::memcpy(&qh, src + 2, 4);  // little-endian host
    for (int i = 0; i < 16; ++i) {
        q[i] = int8_t(((src[6 + i] & 0x0f) | (((qh >> i) & 1u) << 4)) - 16);
        q[i + 16] = int8_t(((src[6 + i] >> 4) | (((qh >> (i + 16)) & 1u) << 4)) - 16);
    }
}

class Reader {
  public:
    Reader(FILE *f, uint64_t size) : f_(f), size_(size) {}
    uint64_t pos() const { return pos_; }
    bool bytes(void *dst, uint64_t n) {
        if (n > size_ - pos_) return false;
        if (n && std::fread(dst, 1, size_t(n), f_) != size_t(n)) return false;
        pos_ += n;
        return true;
    }
    bool skip(uint64_t n) {
        if (n > size_ - pos_) return false;
        if (std::fseek(f_, long(n), SEEK_CUR) != 0) return false;
        pos_ += n;
        return true;
    }
    template <class T>
    bool get(T &v) { return bytes(&v, sizeof(T)); }
    bool str(std::string &s) {
        uint64_t n;
        if (!get(n) || n > size_ - pos_) return false;
        s.resize(size_t(n));
        return bytes(s.data(), n);
    }

  private:
    FILE *f_;
    uint64_t size_;
    uint64_t pos_ = 0;
};

uint64_t scalar_size(uint32_t t) {
    switch (t) {
        case G_U8: case G_I8: case G_BOOL: return 1;
        case G_U16: case G_I16: return 2;
        case G_U32: case G_I32: case G_F32: return 4;
        case G_U64: case G_I64: case G_F64: return 8;
        default: return 0;
    }
}

bool read_scalar(Reader &r, uint32_t t, Value &v) {
    v.type = t;
    switch (t) {
        case G_U8: { uint8_t x; if (!r.get(x)) return false; v.is_int = true; v.u = x; v.i = x; return true; }
        case G_I8: { int8_t x; if (!r.get(x)) return false; v.is_int = true; v.i = x; v.u = uint64_t(x); return true; }
        case G_U16: { uint16_t x; if (!r.get(x)) return false; v.is_int = true; v.u = x; v.i = x; return true; }
        case G_I16: { int16_t x; if (!r.get(x)) return false; v.is_int = true; v.i = x; v.u = uint64_t(x); return true; }
        case G_U32: { uint32_t x; if (!r.get(x)) return false; v.is_int = true; v.u = x; v.i = x; return true; }
        case G_I32: { int32_t x; if (!r.get(x)) return false; v.is_int = true; v.i = x; v.u = uint64_t(x); return true; }
        case G_U64: { uint64_t x; if (!r.get(x)) return false; v.is_int = true; v.u = x; v.i = int64_t(x); return true; }
        case G_I64: { int64_t x; if (!r.get(x)) return false; v.is_int = true; v.i = x; v.u = uint64_t(x); return true; }
        case G_BOOL: { uint8_t x; if (!r.get(x)) return false; v.is_int = true; v.u = x; v.i = x; return true; }
        case G_F32: { float x; if (!r.get(x)) return false; v.is_float = true; v.f = x; return true; }
        case G_F64: { double x; if (!r.get(x)) return false; v.is_float = true; v.f = x; return true; }
        default: return false;
    }
}

// Architectures whose rope pairs dimension j with j + d/2. The pages name
// qwen, qwen2, falcon, phi3 and stablelm among about twenty; gptneox is the
// convention's namesake. Everything else (llama first) pairs 2j with 2j+1.
bool neox_architecture(const std::string &a) {
    static const char *kNeox[] = {"qwen", "qwen2", "falcon", "phi3", "stablelm", "gptneox"};
    for (const char *n : kNeox)
        if (a == n) return true;
    return false;
}

}  // namespace

struct q8l_gguf {
    std::string path;
    FILE *f = nullptr;
    uint32_t version = 0;
    uint64_t file_size = 0;
    uint64_t data_offset = 0;
    uint64_t alignment = 32;
    std::vector<std::pair<std::string, Value>> kv;
    std::map<std::string, size_t> kv_index;
    std::vector<TensorInfo> tensors;
    std::map<std::string, size_t> tensor_index;
    std::string err;
};

namespace {

thread_local std::string g_open_error;

q8l_status fail(q8l_gguf *g, q8l_status st, const std::string &msg) {
    if (g) g->err = msg;
    else g_open_error = msg;
    return st;
}

const Value *find_kv(const q8l_gguf *g, const std::string &key) {
    auto it = g->kv_index.find(key);
    return it == g->kv_index.end() ? nullptr : &g->kv[it->second].second;
}

q8l_status parse(q8l_gguf *g) {
    Reader r(g->f, g->file_size);
    char magic[4];
    if (!r.bytes(magic, 4) || std::memcmp(magic, "GGUF", 4) != 0)
        return fail(g, Q8L_E_FORMAT, "not a GGUF file (bad magic)");
    if (!r.get(g->version)) return fail(g, Q8L_E_FORMAT, "truncated header");
    if (g->version != 2 && g->version != 3)
        return fail(g, Q8L_E_FORMAT, "unsupported GGUF version " + std::to_string(g->version));
    uint64_t n_tensors, n_kv;
    if (!r.get(n_tensors) || !r.get(n_kv)) return fail(g, Q8L_E_FORMAT, "truncated header");
    // every entry takes at least 8 bytes of key/name length: bound the counts
    if (n_kv > g->file_size / 8 || n_tensors > g->file_size / 8)
        return fail(g, Q8L_E_FORMAT, "entry counts exceed the file size");
    g->kv.reserve(size_t(n_kv));
    for (uint64_t i = 0; i < n_kv; ++i) {
        std::string key;
        uint32_t type;
        if (!r.str(key) || !r.get(type)) return fail(g, Q8L_E_FORMAT, "truncated metadata");
        Value v;
        v.type = type;
        if (type == G_STRING) {
            if (!r.str(v.s)) return fail(g, Q8L_E_FORMAT, "truncated metadata string " + key);
        } else if (type == G_ARRAY) {
            if (!r.get(v.arr_type) || !r.get(v.arr_count)) return fail(g, Q8L_E_FORMAT, "truncated array " + key);
            if (v.arr_type == G_STRING) {
                for (uint64_t k = 0; k < v.arr_count; ++k) {
                    uint64_t n;
                    if (!r.get(n) || !r.skip(n)) return fail(g, Q8L_E_FORMAT, "truncated string array " + key);
                }
            } else {
                const uint64_t es = scalar_size(v.arr_type);
                if (!es) return fail(g, Q8L_E_FORMAT, "unsupported array element type in " + key);
                if (v.arr_count > (g->file_size - r.pos()) / es || !r.skip(v.arr_count * es))
                    return fail(g, Q8L_E_FORMAT, "truncated array " + key);
            }
        } else if (!read_scalar(r, type, v)) {
            return fail(g, Q8L_E_FORMAT, "bad metadata value for " + key);
        }
        g->kv_index[key] = g->kv.size();
        g->kv.emplace_back(key, std::move(v));
    }
    if (const Value *a = find_kv(g, "general.alignment")) {
        if (!a->is_int || a->u == 0 || (a->u & (a->u - 1)))
            return fail(g, Q8L_E_FORMAT, "general.alignment must be a power of two");
        g->alignment = a->u;
    }
    g->tensors.reserve(size_t(n_tensors));
    for (uint64_t i = 0; i < n_tensors; ++i) {
        TensorInfo t;
        uint32_t nd;
        if (!r.str(t.name) || !r.get(nd)) return fail(g, Q8L_E_FORMAT, "truncated tensor directory");
        if (nd < 1 || nd > 4) return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " has a bad dimension count");
        t.dims.resize(nd);
        for (uint32_t k = 0; k < nd; ++k)
            if (!r.get(t.dims[k])) return fail(g, Q8L_E_FORMAT, "truncated tensor directory");
        if (!r.get(t.type) || !r.get(t.offset)) return fail(g, Q8L_E_FORMAT, "truncated tensor directory");
        g->tensor_index[t.name] = g->tensors.size();
        g->tensors.push_back(std::move(t));
    }
    const uint64_t a = g->alignment;
    g->data_offset = (r.pos() + a - 1) / a * a;
    if (g->data_offset > g->file_size) return fail(g, Q8L_E_FORMAT, "data region starts past the end of the file");
    // sizes (for the types this library reads) and bounds
    for (TensorInfo &t : g->tensors) {
        uint64_t n = 1;
        for (uint64_t d : t.dims) {
            if (d == 0 || n > (uint64_t(1) << 48) / d) return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " has bad dimensions");
            n *= d;
        }
        if (t.type == kTypeF32) {
            t.file_bytes = t.nbytes = n * 4;
        } else if (q8_family(t.type)) {
            if (t.dims[0] % 32) return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " rows are not whole blocks");
            t.file_bytes = n / 32 * block_bytes(t.type);
            t.native = t.type == kTypeQ5_0 && q5_native_role(t.name) && t.dims[0] >= kQ5NativeMinCols;
            t.nbytes = t.native ? t.file_bytes : n / 32 * 34;
        } else if (k_family(t.type)) {
            if (t.dims[0] % 256) return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " rows are not whole blocks");
            t.file_bytes = t.nbytes = n / 256 * (t.type == kTypeQ4_K ? 144 : 210);
        } else {
            t.file_bytes = t.nbytes = 0;  // other types: listed, not readable (size unknown here)
        }
        if (t.offset % a) return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " is not aligned");
        if (t.offset > g->file_size - g->data_offset || t.file_bytes > g->file_size - g->data_offset - t.offset)
            return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " extends past the end of the file");
    }
    return Q8L_OK;
}

bool get_u(const q8l_gguf *g, const std::string &key, uint64_t &out) {
    const Value *v = find_kv(g, key);
    if (!v || !v->is_int) return false;
    out = v->u;
    return true;
}

bool get_f(const q8l_gguf *g, const std::string &key, double &out) {
    const Value *v = find_kv(g, key);
    if (!v) return false;
    if (v->is_float) out = v->f;
    else if (v->is_int) out = double(v->i);
    else return false;
    return true;
}

}  // namespace

extern "C" {

q8l_status q8l_gguf_open(const char *path, q8l_gguf **out) {
    if (!path || !out) return fail(nullptr, Q8L_E_INVALID_ARG, "path and out are required");
    *out = nullptr;
    FILE *f = std::fopen(path, "rb");
    if (!f) return fail(nullptr, Q8L_E_IO, std::string("cannot open ") + path);
    std::unique_ptr<q8l_gguf> g(new q8l_gguf());
    g->path = path;
    g->f = f;
    // buffered small reads: the header is mostly tiny fields
    std::setvbuf(f, nullptr, _IOFBF, 1 << 16);
    if (std::fseek(f, 0, SEEK_END) != 0) {
        std::fclose(f);
        return fail(nullptr, Q8L_E_IO, "cannot seek");
    }
    g->file_size = uint64_t(std::ftell(f));
    std::rewind(f);
    const q8l_status st = parse(g.get());
    if (st != Q8L_OK) {
        g_open_error = g->err;
        std::fclose(f);
        return st;
    }
    *out = g.release();
    return Q8L_OK;
}

const char *q8l_gguf_open_error(void) { return g_open_error.c_str(); }

const char *q8l_gguf_last_error(const q8l_gguf *g) { return g ? g->err.c_str() : "handle is NULL"; }

void q8l_gguf_close(q8l_gguf *g) {
    if (!g) return;
    if (g->f) std::fclose(g->f);
    delete g;
}

uint32_t q8l_gguf_version(const q8l_gguf *g) { return g ? g->version : 0; }
int64_t q8l_gguf_n_kv(const q8l_gguf *g) { return g ? int64_t(g->kv.size()) : -1; }
int64_t q8l_gguf_n_tensors(const q8l_gguf *g) { return g ? int64_t(g->tensors.size()) : -1; }
uint64_t q8l_gguf_data_offset(const q8l_gguf *g) { return g ? g->data_offset : 0; }
uint64_t q8l_gguf_file_size(const q8l_gguf *g) { return g ? g->file_size : 0; }

q8l_status q8l_gguf_get_number(const q8l_gguf *g, const char *key, double *out) {
    if (!g || !key || !out) return Q8L_E_INVALID_ARG;
    double v;
    if (!get_f(g, key, v))
        return fail(const_cast<q8l_gguf *>(g), Q8L_E_MISSING_KEY, std::string("cannot find ") + key + " in metadata");
    *out = v;
    return Q8L_OK;
}

q8l_status q8l_gguf_get_string(const q8l_gguf *g, const char *key, char *buf, size_t buf_bytes) {
    if (!g || !key || !buf || !buf_bytes) return Q8L_E_INVALID_ARG;
    const Value *v = find_kv(g, key);
    if (!v || v->type != G_STRING)
        return fail(const_cast<q8l_gguf *>(g), Q8L_E_MISSING_KEY, std::string("cannot find ") + key + " in metadata");
    if (v->s.size() + 1 > buf_bytes) return Q8L_E_INVALID_ARG;
    std::memcpy(buf, v->s.c_str(), v->s.size() + 1);
    return Q8L_OK;
}

q8l_status q8l_gguf_config(q8l_gguf *g, int32_t max_seq_len, q8l_config *cfg) {
    if (!g || !cfg || max_seq_len < 1) return Q8L_E_INVALID_ARG;
    auto need = [&](const char *key, uint64_t &v) -> bool {
        if (get_u(g, key, v)) return true;
        fail(g, Q8L_E_MISSING_KEY, std::string("cannot find ") + key + " in metadata");
        return false;
    };
    uint64_t n_layer, n_embd, n_head, n_head_kv, n_ff, rope_dim;
    if (!need("llama.attention.head_count", n_head) || !need("llama.attention.head_count_kv", n_head_kv) ||
        !need("llama.block_count", n_layer) || !need("llama.embedding_length", n_embd) ||
        !need("llama.feed_forward_length", n_ff) || !need("llama.rope.dimension_count", rope_dim))
        return Q8L_E_MISSING_KEY;
    double eps;
    if (!get_f(g, "llama.attention.layer_norm_rms_epsilon", eps))
        return fail(g, Q8L_E_MISSING_KEY, "cannot find llama.attention.layer_norm_rms_epsilon in metadata");
    double theta = 10000.0;
    get_f(g, "llama.rope.freq_base", theta);  // optional
    if (!n_head || n_embd % n_head) return fail(g, Q8L_E_FORMAT, "embedding_length is not a multiple of head_count");
    const uint64_t head_dim = n_embd / n_head;
    if (rope_dim != head_dim)
        return fail(g, Q8L_E_FORMAT, "rope.dimension_count differs from the head width (partial rope)");
    auto it = g->tensor_index.find("token_embd.weight");
    if (it == g->tensor_index.end()) return fail(g, Q8L_E_MISSING_TENSOR, "cannot find token_embd.weight");
    const TensorInfo &emb = g->tensors[it->second];
    if (emb.dims.size() != 2 || emb.dims[0] != n_embd)
        return fail(g, Q8L_E_SHAPE, "token_embd.weight is not [n_vocab, embedding_length]");
    const uint64_t lim = uint64_t(1) << 30;
    if (n_layer > lim || n_embd > lim || n_head > lim || n_head_kv > lim || n_ff > lim || emb.dims[1] > lim)
        return fail(g, Q8L_E_FORMAT, "hyper-parameter out of range");
    std::memset(cfg, 0, sizeof(*cfg));
    cfg->n_layer = int32_t(n_layer);
    cfg->n_embd = int32_t(n_embd);
    cfg->n_head = int32_t(n_head);
    cfg->n_head_kv = int32_t(n_head_kv);
    cfg->head_dim = int32_t(head_dim);
    cfg->n_ff = int32_t(n_ff);
    cfg->n_vocab = int32_t(emb.dims[1]);
    cfg->max_seq_len = max_seq_len;
    cfg->rms_eps = eps;
    cfg->rope_theta = theta;
    // no output.weight: the output layer is the embedding (the pages' tied fallback)
    cfg->tied_output = g->tensor_index.count("output.weight") ? 0 : 1;
    std::string arch;
    if (const Value *a = find_kv(g, "general.architecture"); a && a->type == G_STRING) arch = a->s;
    cfg->rope_type = neox_architecture(arch) ? Q8L_ROPE_NEOX : Q8L_ROPE_NORM;
    return Q8L_OK;
}

int64_t q8l_gguf_find_tensor(const q8l_gguf *g, const char *name) {
    if (!g || !name) return -1;
    auto it = g->tensor_index.find(name);
    return it == g->tensor_index.end() ? -1 : int64_t(it->second);
}

q8l_status q8l_gguf_tensor_info(const q8l_gguf *g, int64_t index, const char **name, int32_t *dtype,
                                int64_t *rows, int64_t *cols, uint64_t *offset, uint64_t *nbytes) {
    if (!g || index < 0 || index >= int64_t(g->tensors.size())) return Q8L_E_INVALID_ARG;
    const TensorInfo &t = g->tensors[size_t(index)];
    if (name) *name = t.name.c_str();
    int64_t r = 1;
    for (size_t k = 1; k < t.dims.size(); ++k) r *= int64_t(t.dims[k]);
    if (rows) *rows = r;
    if (cols) *cols = int64_t(t.dims[0]);
    if (offset) *offset = g->data_offset + t.offset;
    if (nbytes) *nbytes = t.nbytes;
    if (dtype) {
        if (t.type == kTypeF32) *dtype = Q8L_F32;
        else if (t.native) *dtype = Q8L_Q5_0;
        else if (q8_family(t.type)) *dtype = Q8L_Q8_0;
        else if (t.type == kTypeQ4_K) *dtype = Q8L_Q4_K;
        else if (t.type == kTypeQ6_K) *dtype = Q8L_Q6_K;
        else {
            *dtype = -1;
            return fail(const_cast<q8l_gguf *>(g), Q8L_E_FORMAT,
                        "tensor " + t.name + " has type " + std::to_string(t.type) +
                            " (F32, Q8_0, Q4_0, Q5_0, Q4_K and Q6_K are read)");
        }
    }
    return Q8L_OK;
}

int32_t q8l_gguf_tensor_file_type(const q8l_gguf *g, int64_t index) {
    if (!g || index < 0 || index >= int64_t(g->tensors.size())) return -1;
    return int32_t(g->tensors[size_t(index)].type);
}

q8l_status q8l_gguf_read_tensor(q8l_gguf *g, int64_t index, void *host_dst, size_t nbytes) {
    if (!g || !host_dst || index < 0 || index >= int64_t(g->tensors.size())) return Q8L_E_INVALID_ARG;
    const TensorInfo &t = g->tensors[size_t(index)];
    if (t.type != kTypeF32 && !q8_family(t.type) && !k_family(t.type))
        return fail(g, Q8L_E_FORMAT, "tensor " + t.name + " has an unsupported type");
    if (nbytes != t.nbytes) return fail(g, Q8L_E_SHAPE, "tensor " + t.name + ": buffer size differs");
    const uint64_t off = g->data_offset + t.offset;
    if (fseeko(g->f, off_t(off), SEEK_SET) != 0) return fail(g, Q8L_E_IO, "seek failed for " + t.name);
    if (t.type == kTypeF32 || t.type == kTypeQ8_0 || k_family(t.type) || t.native) {
        if (std::fread(host_dst, 1, nbytes, g->f) != nbytes) return fail(g, Q8L_E_IO, "short read for " + t.name);
        return Q8L_OK;
    }
    std::vector<uint8_t> raw(size_t(t.file_bytes));
    if (std::fread(raw.data(), 1, raw.size(), g->f) != raw.size())
        return fail(g, Q8L_E_IO, "short read for " + t.name);
    const uint64_t nblk = t.file_bytes / block_bytes(t.type);
    uint8_t *dst = static_cast<uint8_t *>(host_dst);
    for (uint64_t b = 0; b < nblk; ++b) to_q8_0(t.type, raw.data() + b * block_bytes(t.type), dst + b * 34);
    return Q8L_OK;
}

}  // extern "C"
