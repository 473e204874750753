// runtime.cpp -- host side of the q8l C ABI: model object, tensor binding,
// argument/state checks, workspace layout, kernel sequencing and the decode
// graphs.
//
// The forward is the sequence the page "量化 llama 的一次前向" walks through
// (section "forward：mask 什么时候建"): embedding; per layer attention block and
// MLP block with residuals; final norm on the last position; output layer.
// Kernels per layer: q/k/v (norm + rope + KV write fused), attention,
// o-projection (+ residual), gate/up (norm + SiLU*up fused), down (+ residual).
// Decode with 2..8 attention splits of a small model merges them in the
// o-projection's prologue; more splits take a merge kernel. Short prompts
// split the o and down products over K, and the next norm kernel adds the
// partial sums to the residual.
//
// Decode (one token) runs as a captured HIP graph: every kernel reads the
// position, slot and token from a device-side StepState, so one graph serves
// every step. One graph is captured per power-of-two bucket of attention
// splits (the host knows the cache length, so it picks the bucket); splits
// beyond the keys present exit at once.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/q8l.h"
#include "q8l_internal.h"

namespace q8l {
size_t lmhead_partials_bytes(int V, int K);
__host__ __device__ int attn_chunk(int hd);
}  // namespace q8l

using namespace q8l;

namespace {

const char *kVersion = "q8l 0.1 (gfx950)";

size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct Layout {
    size_t state, counters, rope, tok, kc, vc, x, q, att, h, u, logits, lm_part, attn_part, kpart, total;
    size_t rs, eg_h, el_h;  // prefill activation scaling: row factors, h row / block exponents
    size_t x_alt, part_o;   // decode: second residual row, split-K partials of the fused attention + o
    size_t pf_part;         // prefill attention: partials of key-split query blocks
    int el_stride;          // 32-wide blocks per h row
    size_t kv_layer;  // floats per layer in kc (and vc)
    int max_splits;
};

bool config_ok(const q8l_config *c, std::string *why) {
    auto fail = [&](const char *m) {
        if (why) *why = m;
        return false;
    };
    if (!c) return fail("config is NULL");
    if (c->n_layer < 1 || c->n_embd < 1 || c->n_head < 1 || c->n_head_kv < 1 || c->head_dim < 1 ||
        c->n_ff < 1 || c->n_vocab < 1 || c->max_seq_len < 1)
        return fail("every size in the config must be positive");
    if (c->n_head % c->n_head_kv) return fail("n_head must be a multiple of n_head_kv");
    if (c->n_head / c->n_head_kv > kMaxGroup) return fail("n_head / n_head_kv exceeds 16");
    if (c->head_dim % 8 || c->head_dim > 128) return fail("head_dim must be a multiple of 8 and <= 128");
    if (c->n_embd % 64 || c->n_ff % 64 || (c->n_head * c->head_dim) % 64)
        return fail("n_embd, n_ff and n_head*head_dim must be multiples of 64");
    if (c->n_head_kv > 255) return fail("n_head_kv must be <= 255");
    if (!(c->rms_eps >= 0.0) || !(c->rope_theta > 0.0)) return fail("rms_eps >= 0 and rope_theta > 0 required");
    if (c->rope_type != Q8L_ROPE_NORM && c->rope_type != Q8L_ROPE_NEOX)
        return fail("rope_type must be Q8L_ROPE_NORM or Q8L_ROPE_NEOX");
    return true;
}

Layout make_layout(const q8l_config *c) {
    Layout L{};
    const size_t S = size_t(c->max_seq_len), H = c->n_embd, QD = size_t(c->n_head) * c->head_dim;
    const size_t hd = c->head_dim;
    L.kv_layer = size_t(c->n_head_kv) * S * hd;
    L.max_splits = (c->max_seq_len + attn_chunk(c->head_dim) - 1) / attn_chunk(c->head_dim);
    int pow2 = 1;
    while (pow2 < L.max_splits) pow2 <<= 1;
    L.max_splits = pow2;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = al256(off + bytes);
        return o;
    };
    L.state = take(sizeof(StepState));
    L.counters = take(256 * sizeof(uint32_t));
    L.rope = take(S * (hd / 2) * sizeof(float2));
    L.tok = take(S * sizeof(uint32_t));
    L.kc = take(size_t(c->n_layer) * L.kv_layer * 4);
    L.vc = take(size_t(c->n_layer) * L.kv_layer * 4);
    L.x = take(S * H * 4);
    L.q = take(S * QD * 4);
    L.att = take(S * QD * 4);
    L.h = take(S * size_t(c->n_ff) * 4);
    L.u = take(S * H * 4);  // normalised activations as f16 hi + lo planes (prefill)
    L.logits = take(size_t(c->n_vocab) * 4);
    L.lm_part = take(std::max(lmhead_partials_bytes(c->n_vocab, c->n_embd), size_t(8)));
    L.attn_part = take(size_t(c->n_head) * L.max_splits * (hd + 2) * 4);
    L.kpart = take(size_t(kSplitKMax) * std::max(1, gemm_splitk_max_tokens(int(H))) * H * 4);  // split-K partials
    L.el_stride = c->n_ff / kQK;
    L.rs = take(S * 4);
    L.eg_h = take(S * 4);
    L.el_h = take(S * size_t(L.el_stride));
    L.x_alt = take(H * 4);
    L.part_o = take(size_t(c->n_head_kv) * H * 4);
    // prefill attention key ranges: [n_head][max_seq][kMaxPfSplits][hd + 2]
    L.pf_part = take(attn_prefill_chunk(int(S)) > 0 ? size_t(c->n_head) * S * kMaxPfSplits * (hd + 2) * 4 : 0);
    L.total = off;
    return L;
}

enum Slot { S_ATTN_NORM, S_WQ, S_WK, S_WV, S_WO, S_FFN_NORM, S_WG, S_WU, S_WD, S_NSLOT };
const char *kLayerNames[S_NSLOT] = {"attn_norm", "attn_q", "attn_k", "attn_v", "attn_output",
                                    "ffn_norm", "ffn_gate", "ffn_up", "ffn_down"};

}  // namespace

struct q8l_model {
    q8l_config cfg;
    Dims d;
    Layout lay;
    const uint8_t *tok_embd = nullptr, *output = nullptr;
    const float *out_norm = nullptr;
    bool merge_in_o = false;  // decode o-projection merges 2..8 attention splits in its prologue
    bool fuse_attn_o = false; // one-split decode: attention and o-projection in one kernel (split-K by group)
    std::vector<std::vector<const void *>> layer_ptrs;  // [L][S_NSLOT]
    std::vector<std::vector<int>> fmt;                  // [L][S_NSLOT] WFmt of each matrix
    uint8_t *ws = nullptr;
    size_t ws_bytes = 0;
    bool finalized = false;
    int32_t len = 0;
    std::string err;
    std::map<int, hipGraphExec_t> graphs;  // by (split bucket, steps): graph_key
    std::map<int, hipGraph_t> graph_defs;
    hipStream_t cap = nullptr;
    uint32_t *range_host = nullptr;  // pinned: set by a kernel whose f16-pair split saw a value out of range
    uint32_t *range_dev = nullptr;   // its device address
    // Cache positions [0, kv_checked) hold K and V known to be inside the f16
    // pairs' range (written by a prefill, whose q/k/v kernels check what they
    // write, or checked since); decode steps write unchecked positions, which
    // are checked before a prefill reads them.
    int32_t kv_checked = 0;

    template <typename T>
    T *at(size_t off) const {
        return reinterpret_cast<T *>(ws + off);
    }
    StepState *state() const { return at<StepState>(lay.state); }
    LayerPtrs layer(int l) const {
        const auto &p = layer_ptrs[l];
        LayerPtrs w;
        w.attn_norm = static_cast<const float *>(p[S_ATTN_NORM]);
        w.wq = static_cast<const uint8_t *>(p[S_WQ]);
        w.wk = static_cast<const uint8_t *>(p[S_WK]);
        w.wv = static_cast<const uint8_t *>(p[S_WV]);
        w.wo = static_cast<const uint8_t *>(p[S_WO]);
        w.ffn_norm = static_cast<const float *>(p[S_FFN_NORM]);
        w.wg = static_cast<const uint8_t *>(p[S_WG]);
        w.wu = static_cast<const uint8_t *>(p[S_WU]);
        w.wd = static_cast<const uint8_t *>(p[S_WD]);
        const auto &f = fmt[l];
        w.fq = f[S_WQ]; w.fk = f[S_WK]; w.fv = f[S_WV]; w.fo = f[S_WO];
        w.fg = f[S_WG]; w.fu = f[S_WU]; w.fd = f[S_WD];
        return w;
    }
    float *kc(int l) const { return at<float>(lay.kc) + size_t(l) * lay.kv_layer; }
    float *vc(int l) const { return at<float>(lay.vc) + size_t(l) * lay.kv_layer; }
};

namespace {

q8l_status fail(q8l_model *m, q8l_status st, const std::string &msg) {
    if (m) m->err = msg;
    return st;
}

q8l_status hip_fail(q8l_model *m, hipError_t e, const char *what) {
    return fail(m, Q8L_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define Q8L_HIP(m, expr, what)                              \
    do {                                                    \
        hipError_t e_ = (expr);                             \
        if (e_ != hipSuccess) return hip_fail((m), e_, what); \
    } while (0)

// The q/k/v ... down kernels of one layer plus the attention, for T tokens.
hipError_t enqueue_layers(q8l_model *m, int T, int kv_len_prefill, int decode_splits,
                          hipStream_t s) {
    const Dims &d = m->d;
    const int QD = d.nh * d.hd;
    StepState *st = m->state();
    float *x = m->at<float>(m->lay.x), *q = m->at<float>(m->lay.q);
    float *att = m->at<float>(m->lay.att), *h = m->at<float>(m->lay.h);
    const float2 *rope = m->at<float2>(m->lay.rope);
    hipError_t e;
    const bool gemm = T >= kGemmMinTokens;  // MFMA matrix-matrix path for prompts
    _Float16 *u = m->at<_Float16>(m->lay.u);
    _Float16 *att_s = m->at<_Float16>(m->lay.att), *h_s = m->at<_Float16>(m->lay.h);
    float *kpart = m->at<float>(m->lay.kpart);
    int pend = 0;  // split-K partial sums not yet added to x (the next norm kernel adds them)
    // Decode residual: two rows. A kernel that adds split-K partials (of the
    // fused attention + o-projection) to the residual reads xr[cur] and its
    // workgroup 0 writes the sum to xr[cur ^ 1] (the others still read
    // xr[cur]); cur then flips. Prefill keeps x.
    float *xr[2] = {x, m->at<float>(m->lay.x_alt)};
    int cur = 0;
    PartSrc dpend;  // decode partials not yet added to xr[cur]
    auto take_pending = [&]() {
        PartSrc p = dpend;
        if (p.n > 0) {
            p.xout = xr[cur ^ 1];
            cur ^= 1;
        }
        dpend = PartSrc{};
        return p;
    };
    // Activation scaling of the f16-pair planes (ActScale): the normalised
    // rows carry per-row factors, h per-(row, block) exponents from the
    // gate/up epilogue; q/k/v, the attention output and f32 inputs split
    // on the way are range-checked.
    float *rs = m->at<float>(m->lay.rs);
    int *eg_h = m->at<int>(m->lay.eg_h);
    int8_t *el_h = m->at<int8_t>(m->lay.el_h);
    ActScale sc_u, sc_o, sc_h_out, sc_h_in;
    sc_u.rs = rs;
    sc_u.range_flag = sc_o.range_flag = sc_h_out.range_flag = sc_h_in.range_flag = m->range_dev;
    sc_h_out.rs = rs;
    sc_h_out.eg_out = eg_h;
    sc_h_out.el_out = el_h;
    sc_h_out.el_stride = m->lay.el_stride;
    sc_h_in.eg = eg_h;
    sc_h_in.el = el_h;
    sc_h_in.el_stride = m->lay.el_stride;
    // Prefill x += A W^T for a Q8_0 matrix of H rows: split over K when the
    // plain grid would be small (the partial sums wait in kpart).
    auto gemm_accumulate = [&](const uint8_t *W, int K, const _Float16 *A, const ActScale &sc,
                               int fmt) -> hipError_t {
        const int sk = gemm_splitk(d.H, K, T);
        pend = sk > 1 ? sk : 0;
        return sk > 1 ? launch_gemm_part(W, d.H, K, A, T, sk, kpart, s, sc, fmt)
                      : launch_gemm_matmul(W, d.H, K, A, true, T, 1, x, s, sc, fmt);
    };
    for (int l = 0; l < m->cfg.n_layer; ++l) {
        const LayerPtrs w = m->layer(l);
        if (gemm) {
            if ((e = launch_rms_split(x, T, d.H, w.attn_norm, d.eps, u, kpart, pend, s, rs)) != hipSuccess) return e;
            pend = 0;
            if ((e = launch_gemm_qkv(d, w, u, st, rope, q, m->kc(l), m->vc(l), T, s, sc_u)) != hipSuccess) return e;
        } else {
            // a decode step's first layer dequantizes the token's embedding itself
            const uint8_t *emb = (T == 1 && l == 0) ? m->tok_embd : nullptr;
            float *xin = xr[cur];
            const PartSrc ps = take_pending();
            if ((e = launch_qkv(d, w, xin, st, rope, q, m->kc(l), m->vc(l), T, s, emb, emb ? xin : nullptr, ps,
                                m->range_dev)) != hipSuccess)
                return e;
        }
        if (d.rope_neox && (e = launch_rope_neox(d, st, rope, q, m->kc(l), T, s, m->range_dev)) != hipSuccess)
            return e;
        if (T == 1) {
            bool continue_ffn = false;
            AttnDecodeArgs a;
            a.q = q; a.kc = m->kc(l); a.vc = m->vc(l);
            a.part = m->at<float>(m->lay.attn_part);
            a.st = st; a.kv_len_arg = -1; a.kv_stride = d.max_seq;
            a.nh = d.nh; a.nkv = d.nkv; a.hd = d.hd; a.n_splits = decode_splits;
            a.scale = 1.0f / sqrtf(float(d.hd));
            a.o = decode_splits == 1 ? att : nullptr;  // one split: the attention kernel normalises
            if (decode_splits == 1 && !kq_format(w.fo) && m->fuse_attn_o) {
                // one kernel; its partial sums wait for the gate/up kernel's prologue
                float *part_o = m->at<float>(m->lay.part_o);
                if ((e = launch_attn_o(a, w.wo, d.H, part_o, s, w.fo)) != hipSuccess) return e;
                dpend.part = part_o;
                dpend.n = d.nkv;
                dpend.stride = d.H;
                continue_ffn = true;
            }
            if (!continue_ffn) {
                float *xo = xr[cur];
                // a few splits of a small model: the o-projection merges them in its prologue (no merge node)
                const bool merge_o = w.fo == F_Q8_0 && m->merge_in_o && oproj_merges(d, decode_splits);
                if ((e = launch_attn_decode(a, s)) != hipSuccess) return e;
                if (decode_splits > 1 && !merge_o &&
                    (e = launch_attn_combine(a.part, decode_splits, 0, d.nh, d.hd, att, st, s)) != hipSuccess)
                    return e;
                e = kq_format(w.fo) ? launch_kq_gemv(w.fo, w.wo, d.H, QD, att, 1, xo, s)
                    : merge_o       ? launch_oproj_merged(w.wo, d.H, QD, a.part, decode_splits, d.hd, st, xo, s)
                                    : launch_matmul(w.wo, d.H, QD, att, 1, nullptr, d.eps, 1, xo, s, w.fo);
                if (e != hipSuccess) return e;
            }
        } else {
            AttnPrefillArgs a;
            a.q = q; a.kc = m->kc(l); a.vc = m->vc(l); a.o = att;
            a.o_split = gemm ? att_s : nullptr;  // the o-projection GEMM reads f16 hi + lo
            a.T = T; a.kv_len = kv_len_prefill; a.kv_stride = d.max_seq;
            a.nh = d.nh; a.nkv = d.nkv; a.hd = d.hd; a.scale = 1.0f / sqrtf(float(d.hd));
            a.range_flag = m->range_dev;
            a.pf_chunk = attn_prefill_chunk(kv_len_prefill);   // long prompts: key ranges in parallel
            a.pf_part = a.pf_chunk > 0 ? m->at<float>(m->lay.pf_part) : nullptr;
            if ((e = launch_attn_prefill(a, s)) != hipSuccess) return e;
            if (kq_format(w.fo))
                e = gemm ? launch_gemm_kq(w.fo, w.wo, d.H, QD, att_s, true, T, 1, x, s, sc_o)
                         : launch_gemm_kq(w.fo, w.wo, d.H, QD, att, false, T, 1, x, s, sc_o);
            else if (gemm)
                e = gemm_accumulate(w.wo, QD, att_s, sc_o, w.fo);
            else
                e = launch_matmul(w.wo, d.H, QD, att, T, nullptr, d.eps, 1, x, s, w.fo);
            if (e != hipSuccess) return e;
        }
        if (gemm) {
            if ((e = launch_rms_split(x, T, d.H, w.ffn_norm, d.eps, u, kpart, pend, s, rs, eg_h, el_h,
                                      m->lay.el_stride)) != hipSuccess)
                return e;
            pend = 0;
            if ((e = launch_gemm_gateup(d, w, u, h_s, T, s, sc_h_out)) != hipSuccess) return e;
            e = kq_format(w.fd) ? launch_gemm_kq(w.fd, w.wd, d.H, d.F, h_s, true, T, 1, x, s, sc_h_in)
                                : gemm_accumulate(w.wd, d.F, h_s, sc_h_in, w.fd);
        } else {
            const float *xin = xr[cur];
            const PartSrc ps = take_pending();
            if ((e = launch_gateup(d, w, xin, h, T, s, ps)) != hipSuccess) return e;
            float *xd = xr[cur];
            if (!kq_format(w.fd))
                e = launch_matmul(w.wd, d.H, d.F, h, T, nullptr, d.eps, 1, xd, s, w.fd);
            else if (T == 1)
                e = launch_kq_gemv(w.fd, w.wd, d.H, d.F, h, 1, xd, s);
            else
                e = launch_gemm_kq(w.fd, w.wd, d.H, d.F, h, false, T, 1, xd, s, sc_o);
        }
        if (e != hipSuccess) return e;
    }
    if (pend > 0 && (e = launch_rms_split(x, T, d.H, nullptr, d.eps, nullptr, kpart, pend, s)) != hipSuccess)
        return e;
    const uint8_t *wout = m->cfg.tied_output ? m->tok_embd : m->output;
    PartSrc ps = dpend;  // (none: every layer ends with a plain down projection)
    if ((e = launch_lmhead(d, wout, m->out_norm, xr[cur] + size_t(T - 1) * d.H, st,
                           m->at<float>(m->lay.lm_part), s, ps)) != hipSuccess)
        return e;
    return launch_argmax_finish(d, m->at<float>(m->lay.lm_part), st, s);
}

// Decode graph variant for a cache length: the power-of-two number of
// attention splits that covers it.
int split_bucket(const q8l_model *m, int kv_len) {
    const int need = (kv_len + attn_chunk(m->d.hd) - 1) / attn_chunk(m->d.hd);
    int b = 1;
    while (b < need) b <<= 1;
    return std::min(b, m->lay.max_splits);
}

// Decode graphs hold 1, 2, 4, ... kMaxGraphSteps consecutive steps of one
// split bucket (each step's kernels read the position, slot and token that
// the previous step's argmax kernel advanced on the device).
constexpr int kMaxGraphSteps = 16;
int graph_key(int bucket, int steps) { return bucket * 64 + steps; }

q8l_status decode_graph(q8l_model *m, int bucket, hipGraphExec_t *out, int steps = 1) {
    const int key = graph_key(bucket, steps);
    auto it = m->graphs.find(key);
    if (it != m->graphs.end()) {
        *out = it->second;
        return Q8L_OK;
    }
    if (!m->cap) Q8L_HIP(m, hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking), "hipStreamCreate");
    Q8L_HIP(m, hipStreamBeginCapture(m->cap, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
    // (no embedding kernel: the first layer's q/k/v kernel reads the embedding)
    hipError_t e = hipSuccess;
    for (int k = 0; k < steps && e == hipSuccess; ++k) e = enqueue_layers(m, 1, -1, bucket, m->cap);
    hipGraph_t g = nullptr;
    hipError_t e2 = hipStreamEndCapture(m->cap, &g);
    if (e != hipSuccess) {
        if (g) hipGraphDestroy(g);
        return hip_fail(m, e, "capturing the decode step");
    }
    if (e2 != hipSuccess) return hip_fail(m, e2, "hipStreamEndCapture");
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        hipGraphDestroy(g);
        return hip_fail(m, e, "hipGraphInstantiate");
    }
    m->graphs[key] = ex;
    m->graph_defs[key] = g;
    *out = ex;
    return Q8L_OK;
}

const char *dtype_name(int t) {
    return t == Q8L_F32 ? "F32" : t == Q8L_Q8_0 ? "Q8_0" : t == Q8L_Q4_K ? "Q4_K" : t == Q8L_Q6_K ? "Q6_K"
         : t == Q8L_Q5_0 ? "Q5_0" : "unknown";
}

bool parse_layer_name(const char *name, int *layer, int *slot) {
    if (std::strncmp(name, "blk.", 4) != 0) return false;
    const char *p = name + 4;
    if (*p < '0' || *p > '9') return false;
    long v = 0;
    while (*p >= '0' && *p <= '9') {
        v = v * 10 + (*p - '0');
        if (v > 1000000) return false;
        ++p;
    }
    if (*p != '.') return false;
    ++p;
    for (int s = 0; s < S_NSLOT; ++s) {
        const size_t n = std::strlen(kLayerNames[s]);
        if (std::strncmp(p, kLayerNames[s], n) == 0 && std::strcmp(p + n, ".weight") == 0) {
            *layer = int(v);
            *slot = s;
            return true;
        }
    }
    return false;
}

// The index_pos / cache-length contract, checked before any change.
q8l_status check_positions(q8l_model *m, int32_t T, int32_t index_pos, int32_t *eff_len) {
    const int32_t S = m->cfg.max_seq_len;
    if (int64_t(index_pos) + T > S)
        return fail(m, Q8L_E_POS_RANGE,
                    "index_pos + n_tokens = " + std::to_string(int64_t(index_pos) + T) +
                        " exceeds the rope table length " + std::to_string(S));
    const int32_t len = index_pos == 0 ? 0 : m->len;
    if (T > 1 && index_pos != len)
        return fail(m, Q8L_E_POS_MISMATCH,
                    "index_pos " + std::to_string(index_pos) + " != cached positions " +
                        std::to_string(len) + " with " + std::to_string(T) + " tokens");
    if (int64_t(len) + T > S)
        return fail(m, Q8L_E_KV_FULL, "cached positions " + std::to_string(len) + " + " +
                                          std::to_string(T) + " exceed " + std::to_string(S));
    *eff_len = len;
    return Q8L_OK;
}

q8l_status set_state(q8l_model *m, int pos, int slot, int T, int advance, float *logits,
                     uint32_t *argmax, uint32_t *ids, const uint32_t *tokens, hipStream_t s) {
    SetStateArgs a{};
    a.pos = pos; a.slot = slot; a.T = T; a.step = 0; a.advance = advance;
    a.logits_out = logits; a.argmax_out = argmax; a.ids_out = ids;
    a.set_header = 1;
    const int n = tokens ? T : 0;
    int off = 0;
    do {
        a.tok_offset = off;
        a.tok_count = std::min(n - off, kInlineTokens);
        if (a.tok_count > 0) std::memcpy(a.tokens, tokens + off, sizeof(uint32_t) * a.tok_count);
        Q8L_HIP(m, launch_set_state(a, m->state(), m->at<uint32_t>(m->lay.tok), s), "set_state");
        a.set_header = 0;
        off += std::max(a.tok_count, 0);
    } while (off < n);
    return Q8L_OK;
}

// A prefill kernel of an earlier call split a value outside the f16 pairs'
// range into a pair (see ActScale): reported once, by the next call.
q8l_status range_check(q8l_model *m) {
    if (!m->range_host || __atomic_load_n(m->range_host, __ATOMIC_ACQUIRE) == 0) return Q8L_OK;
    __atomic_store_n(m->range_host, 0u, __ATOMIC_RELEASE);
    return fail(m, Q8L_E_RANGE,
                "an earlier prefill split a q/k/v or input value of magnitude >= 32768 (or not finite) into an "
                "f16 pair: its logits are not exact");
}

}  // namespace

extern "C" {

const char *q8l_version(void) { return kVersion; }

size_t q8l_workspace_bytes(const q8l_config *cfg) {
    if (!config_ok(cfg, nullptr)) return 0;
    return make_layout(cfg).total;
}

q8l_status q8l_create(const q8l_config *cfg, q8l_model **out) {
    if (!out) return Q8L_E_INVALID_ARG;
    *out = nullptr;
    std::string why;
    if (!config_ok(cfg, &why)) return Q8L_E_INVALID_ARG;
    q8l_model *m = new q8l_model();
    m->cfg = *cfg;
    m->d.H = cfg->n_embd; m->d.nh = cfg->n_head; m->d.nkv = cfg->n_head_kv; m->d.hd = cfg->head_dim;
    m->d.F = cfg->n_ff; m->d.V = cfg->n_vocab; m->d.max_seq = cfg->max_seq_len;
    m->d.eps = float(cfg->rms_eps);
    m->d.rope_neox = cfg->rope_type == Q8L_ROPE_NEOX ? 1 : 0;
    m->lay = make_layout(cfg);
    // the merged attention row is staged whole in LDS (as the o-projection GEMV stages rows of <= 150 pairs)
    m->merge_in_o = (cfg->n_head * cfg->head_dim / kPairWeights) * 68 * 4 <= 40 * 1024;
    // every workgroup of the kernel after the fused attention + o-projection
    // reads the n_head_kv partial rows: only while they are a few KB
    m->fuse_attn_o = attn_o_fits(m->d) && size_t(cfg->n_head_kv) * cfg->n_embd * 4 <= kFuseAttnOMaxBytes;
    m->layer_ptrs.assign(cfg->n_layer, std::vector<const void *>(S_NSLOT, nullptr));
    m->fmt.assign(cfg->n_layer, std::vector<int>(S_NSLOT, F_Q8_0));
    *out = m;
    return Q8L_OK;
}

q8l_status q8l_bind_tensor(q8l_model *m, const char *name, q8l_dtype dtype, int64_t rows,
                           int64_t cols, const void *dev_ptr, size_t nbytes) {
    if (!m) return Q8L_E_INVALID_ARG;
    if (m->finalized) return fail(m, Q8L_E_NOT_FINALIZED, "weights are fixed after finalize");
    if (!name || !dev_ptr) return fail(m, Q8L_E_INVALID_ARG, "name and dev_ptr must not be NULL");
    if (reinterpret_cast<uintptr_t>(dev_ptr) & 15)
        return fail(m, Q8L_E_INVALID_ARG, std::string(name) + ": pointer not 16-byte aligned");
    const q8l_config &c = m->cfg;
    const int64_t H = c.n_embd, QD = int64_t(c.n_head) * c.head_dim, KVD = int64_t(c.n_head_kv) * c.head_dim;
    int64_t er = 0, ec = 0;
    q8l_dtype et = Q8L_Q8_0;
    const void **slot = nullptr;
    int layer = -1, s = -1;
    if (std::strcmp(name, "token_embd.weight") == 0) {
        er = c.n_vocab; ec = H; slot = reinterpret_cast<const void **>(&m->tok_embd);
    } else if (std::strcmp(name, "output.weight") == 0) {
        if (c.tied_output) return fail(m, Q8L_E_INVALID_ARG, "output.weight given for a tied model");
        er = c.n_vocab; ec = H; slot = reinterpret_cast<const void **>(&m->output);
    } else if (std::strcmp(name, "output_norm.weight") == 0) {
        er = 1; ec = H; et = Q8L_F32; slot = reinterpret_cast<const void **>(&m->out_norm);
    } else if (parse_layer_name(name, &layer, &s)) {
        if (layer >= c.n_layer) return fail(m, Q8L_E_INVALID_ARG, std::string(name) + ": layer out of range");
        switch (s) {
            case S_ATTN_NORM: case S_FFN_NORM: er = 1; ec = H; et = Q8L_F32; break;
            case S_WQ: er = QD; ec = H; break;
            case S_WK: case S_WV: er = KVD; ec = H; break;
            case S_WO: er = H; ec = QD; break;
            case S_WG: case S_WU: er = c.n_ff; ec = H; break;
            case S_WD: er = H; ec = c.n_ff; break;
        }
        slot = &m->layer_ptrs[layer][s];
    } else {
        return fail(m, Q8L_E_INVALID_ARG, std::string("unknown tensor name ") + name);
    }
    // attn_output and ffn_down may also be Q4_K / Q6_K (rows of whole 256-weight
    // blocks); every projection of a layer may be Q5_0
    const bool kquant_ok = layer >= 0 && (s == S_WO || s == S_WD) && ec % kQKK == 0;
    const bool q5_ok = layer >= 0 && (s == S_WQ || s == S_WK || s == S_WV || s == S_WO || s == S_WG || s == S_WU ||
                                      s == S_WD);
    if (kquant_ok && (dtype == Q8L_Q4_K || dtype == Q8L_Q6_K)) et = dtype;
    if (q5_ok && dtype == Q8L_Q5_0) et = dtype;
    const int ef = et == Q8L_Q4_K ? F_Q4_K : et == Q8L_Q6_K ? F_Q6_K : et == Q8L_Q5_0 ? F_Q5_0 : F_Q8_0;
    const size_t want = et == Q8L_F32 ? size_t(er * ec * 4) : size_t(er * fmt_row_bytes(ef, ec));
    if (dtype != et || rows != er || cols != ec || nbytes != want) {
        char buf[320];
        const char *allowed = et != Q8L_Q8_0 ? dtype_name(et)
                              : kquant_ok && q5_ok ? "Q8_0, Q5_0, Q4_K or Q6_K"
                              : kquant_ok          ? "Q8_0, Q4_K or Q6_K"
                              : q5_ok              ? "Q8_0 or Q5_0"
                                                   : "Q8_0";
        std::snprintf(buf, sizeof buf, "%s: expected %s [%lld, %lld] (%zu bytes), got %s [%lld, %lld] (%zu bytes)",
                      name, allowed, (long long)er, (long long)ec, want, dtype_name(dtype), (long long)rows,
                      (long long)cols, nbytes);
        return fail(m, Q8L_E_SHAPE, buf);
    }
    *slot = dev_ptr;
    if (layer >= 0 && et != Q8L_F32) m->fmt[layer][s] = ef;
    return Q8L_OK;
}

q8l_status q8l_bind_workspace(q8l_model *m, void *dev_ptr, size_t nbytes) {
    if (!m) return Q8L_E_INVALID_ARG;
    if (m->finalized) return fail(m, Q8L_E_NOT_FINALIZED, "workspace is fixed after finalize");
    if (!dev_ptr || (reinterpret_cast<uintptr_t>(dev_ptr) & 255))
        return fail(m, Q8L_E_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
    if (nbytes < m->lay.total)
        return fail(m, Q8L_E_INVALID_ARG, "workspace too small: need " + std::to_string(m->lay.total) +
                                              " bytes, got " + std::to_string(nbytes));
    m->ws = static_cast<uint8_t *>(dev_ptr);
    m->ws_bytes = nbytes;
    return Q8L_OK;
}

q8l_status q8l_finalize(q8l_model *m, void *stream) {
    if (!m) return Q8L_E_INVALID_ARG;
    if (m->finalized) return Q8L_OK;
    if (!m->tok_embd) return fail(m, Q8L_E_MISSING_TENSOR, "cannot find token_embd.weight");
    for (int l = 0; l < m->cfg.n_layer; ++l)
        for (int s = 0; s < S_NSLOT; ++s)
            if (!m->layer_ptrs[l][s])
                return fail(m, Q8L_E_MISSING_TENSOR, "cannot find blk." + std::to_string(l) + "." +
                                                         kLayerNames[s] + ".weight");
    if (!m->out_norm) return fail(m, Q8L_E_MISSING_TENSOR, "cannot find output_norm.weight");
    if (!m->cfg.tied_output && !m->output) return fail(m, Q8L_E_MISSING_TENSOR, "cannot find output.weight");
    if (!m->ws) return fail(m, Q8L_E_MISSING_TENSOR, "no workspace bound");
    for (int l = 0; l < m->cfg.n_layer; ++l)   // gate and up run as one product
        if (m->fmt[l][S_WG] != m->fmt[l][S_WU])
            return fail(m, Q8L_E_SHAPE, "blk." + std::to_string(l) + ": ffn_gate and ffn_up must share a format");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Q8L_HIP(m, hipMemsetAsync(m->ws + m->lay.state, 0, m->lay.rope - m->lay.state, s), "clearing state");
    Q8L_HIP(m, launch_rope_table(m->at<float2>(m->lay.rope), m->cfg.max_seq_len, m->cfg.head_dim,
                                 m->cfg.rope_theta, s),
            "building the rope table");
    if (!m->range_host) {
        void *p = nullptr;
        Q8L_HIP(m, hipHostMalloc(&p, 64, hipHostMallocMapped), "hipHostMalloc");
        m->range_host = static_cast<uint32_t *>(p);
        *m->range_host = 0;
        void *dp = nullptr;
        Q8L_HIP(m, hipHostGetDevicePointer(&dp, p, 0), "hipHostGetDevicePointer");
        m->range_dev = static_cast<uint32_t *>(dp);
    }
    m->len = 0;
    m->finalized = true;
    return Q8L_OK;
}

q8l_status q8l_forward(q8l_model *m, const uint32_t *tokens_host, int32_t n_tokens,
                       int32_t index_pos, float *logits_dev, uint32_t *argmax_dev, void *stream) {
    if (!m) return Q8L_E_INVALID_ARG;
    if (n_tokens < 1 || !tokens_host || index_pos < 0 || !logits_dev)
        return fail(m, Q8L_E_INVALID_ARG, "need n_tokens >= 1, tokens, index_pos >= 0 and logits_dev");
    for (int32_t i = 0; i < n_tokens; ++i)
        if (tokens_host[i] >= uint32_t(m->cfg.n_vocab))
            return fail(m, Q8L_E_INVALID_ARG, "token id " + std::to_string(tokens_host[i]) +
                                                  " at " + std::to_string(i) + " >= n_vocab");
    int32_t len;
    q8l_status st = check_positions(m, n_tokens, index_pos, &len);
    if (st != Q8L_OK) return st;
    if (!m->finalized) return fail(m, Q8L_E_NOT_FINALIZED, "forward before finalize");
    if ((st = range_check(m)) != Q8L_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int T = n_tokens;
    m->kv_checked = std::min(m->kv_checked, len);   // positions past len are dropped
    if (T == 1) {
        hipGraphExec_t g;
        if ((st = decode_graph(m, split_bucket(m, len + 1), &g)) != Q8L_OK) return st;
        if ((st = set_state(m, index_pos, len, 1, 0, logits_dev, argmax_dev, nullptr, tokens_host, s)) != Q8L_OK)
            return st;
        Q8L_HIP(m, hipGraphLaunch(g, s), "hipGraphLaunch");
    } else {
        if ((st = set_state(m, index_pos, len, T, 0, logits_dev, argmax_dev, nullptr, tokens_host, s)) != Q8L_OK)
            return st;
        Q8L_HIP(m, launch_embed(m->tok_embd, m->d.H, m->d.V, m->state(), m->at<uint32_t>(m->lay.tok), T, 0,
                                m->at<float>(m->lay.x), s),
                "embedding");
        // the prefill's attention reads the cached positions as f16 pairs:
        // check those a decode step wrote (its own q/k/v are checked as written)
        Q8L_HIP(m, launch_kv_range(m->kc(0), m->vc(0), m->lay.kv_layer, m->cfg.n_layer, m->d.nkv, m->d.max_seq,
                                   m->d.hd, m->kv_checked, len, m->range_dev, s),
                "cache range check");
        Q8L_HIP(m, enqueue_layers(m, T, len + T, 0, s), "prefill");
        m->kv_checked = len + T;
    }
    m->len = len + T;
    m->err.clear();
    return Q8L_OK;
}

q8l_status q8l_generate(q8l_model *m, const uint32_t *token_dev, int32_t index_pos,
                        int32_t n_steps, uint32_t *ids_dev, float *logits_dev, void *stream) {
    if (!m) return Q8L_E_INVALID_ARG;
    if (!token_dev || !ids_dev || n_steps < 1 || index_pos < 0)
        return fail(m, Q8L_E_INVALID_ARG, "need token_dev, ids_dev, n_steps >= 1, index_pos >= 0");
    const int32_t S = m->cfg.max_seq_len;
    if (int64_t(index_pos) + n_steps > S)
        return fail(m, Q8L_E_POS_RANGE, "index_pos + n_steps exceeds the rope table length");
    const int32_t len = index_pos == 0 ? 0 : m->len;
    if (int64_t(len) + n_steps > S) return fail(m, Q8L_E_KV_FULL, "cache would overflow");
    if (!m->finalized) return fail(m, Q8L_E_NOT_FINALIZED, "generate before finalize");
    if (q8l_status rc = range_check(m); rc != Q8L_OK) return rc;
    m->kv_checked = std::min(m->kv_checked, len);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // runs of steps in one split bucket, as graphs of power-of-two step counts
    std::vector<hipGraphExec_t> gs;
    for (int k = 0; k < n_steps;) {
        const int b = split_bucket(m, len + k + 1);
        int run = 1;
        while (k + run < n_steps && run < kMaxGraphSteps && split_bucket(m, len + k + run + 1) == b) ++run;
        int p = 1;
        while (p * 2 <= run) p *= 2;
        hipGraphExec_t g = nullptr;
        q8l_status st = decode_graph(m, b, &g, p);
        if (st != Q8L_OK) return st;
        gs.push_back(g);
        k += p;
    }
    float *lg = logits_dev ? logits_dev : m->at<float>(m->lay.logits);
    q8l_status st = set_state(m, index_pos, len, 1, 1, lg, nullptr, ids_dev, nullptr, s);
    if (st != Q8L_OK) return st;
    Q8L_HIP(m, hipMemcpyAsync(&m->state()->token, token_dev, sizeof(uint32_t), hipMemcpyDeviceToDevice, s),
            "token copy");
    for (hipGraphExec_t g : gs) Q8L_HIP(m, hipGraphLaunch(g, s), "hipGraphLaunch");
    m->len = len + n_steps;
    m->err.clear();
    return Q8L_OK;
}

q8l_status q8l_time_decode_kernels(q8l_model *m, int32_t reps, float *ms_out, void *stream) {
    if (!m) return Q8L_E_INVALID_ARG;
    if (!m->finalized) return fail(m, Q8L_E_NOT_FINALIZED, "timing before finalize");
    if (reps < 1 || !ms_out || m->len + 1 > m->cfg.max_seq_len)
        return fail(m, Q8L_E_INVALID_ARG, "need reps >= 1, ms_out, and a free cache slot");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Dims &d = m->d;
    const int QD = d.nh * d.hd;
    const int kv_len = m->len + 1;
    q8l_status st = set_state(m, m->len, m->len, 1, 0, m->at<float>(m->lay.logits), nullptr, nullptr,
                              nullptr, s);
    if (st != Q8L_OK) return st;
    StepState *S = m->state();
    float *x = m->at<float>(m->lay.x), *q = m->at<float>(m->lay.q);
    float *h = m->at<float>(m->lay.h);
    const uint8_t *wout = m->cfg.tied_output ? m->tok_embd : m->output;
    const int n_splits = split_bucket(m, kv_len);
    // as in the step: with one split the attention and the o-projection are
    // one kernel, and gate/up adds its partial sums to the residual first
    const bool fused = n_splits == 1 && m->fuse_attn_o && !kq_format(m->layer(0).fo);
    PartSrc ps_gu;
    if (fused) {
        ps_gu.part = m->at<float>(m->lay.part_o);
        ps_gu.n = d.nkv;
        ps_gu.stride = d.H;
        ps_gu.xout = m->at<float>(m->lay.x_alt);
    }
    int rep = 0;  // launches of the current kind so far: layer rep mod n_layer
    auto launch = [&](int kind) -> hipError_t {
        const int l = rep++ % m->cfg.n_layer;
        const LayerPtrs w = m->layer(l);
        AttnDecodeArgs a;
        a.q = q; a.kc = m->kc(l); a.vc = m->vc(l);
        a.part = m->at<float>(m->lay.attn_part);
        a.st = S; a.kv_len_arg = -1; a.kv_stride = d.max_seq;
        a.nh = d.nh; a.nkv = d.nkv; a.hd = d.hd; a.n_splits = n_splits;
        a.scale = 1.0f / sqrtf(float(d.hd));
        a.o = a.n_splits == 1 ? m->at<float>(m->lay.att) : nullptr;
        switch (kind) {
            case 0:  // the step has no embedding kernel: these launches only warm the
                     // GPU up for the timed kinds (reported as -1)
                return launch_qkv(d, w, x, S, m->at<float2>(m->lay.rope), q, m->kc(l), m->vc(l), 1, s);
            case 1:  // q/k/v as every layer but the first runs it (that one also reads the embedding)
                return launch_qkv(d, w, x, S, m->at<float2>(m->lay.rope), q, m->kc(l), m->vc(l), 1, s);
            case 2:
                if (fused && !kq_format(w.fo))
                    return launch_attn_o(a, w.wo, d.H, m->at<float>(m->lay.part_o), s, w.fo);
                return launch_attn_decode(a, s);
            case 3:
                if (kq_format(w.fo)) return launch_kq_gemv(w.fo, w.wo, d.H, QD, m->at<float>(m->lay.att), 1, x, s);
                if (w.fo == F_Q8_0 && m->merge_in_o && oproj_merges(d, a.n_splits))  // as in the step
                    return launch_oproj_merged(w.wo, d.H, QD, a.part, a.n_splits, d.hd, S, x, s);
                return launch_matmul(w.wo, d.H, QD, m->at<float>(m->lay.att), 1, nullptr, d.eps, 1, x, s, w.fo);
            case 4: return launch_gateup(d, w, x, h, 1, s, ps_gu);
            case 5:
                if (kq_format(w.fd)) return launch_kq_gemv(w.fd, w.wd, d.H, d.F, h, 1, x, s);
                return launch_matmul(w.wd, d.H, d.F, h, 1, nullptr, d.eps, 1, x, s, w.fd);
            case 6: return launch_lmhead(d, wout, m->out_norm, x, S, m->at<float>(m->lay.lm_part), s);
            case 7: return launch_argmax_finish(d, m->at<float>(m->lay.lm_part), S, s);
            default: return launch_noop(s);
        }
    };
    constexpr int kKinds = 9;
    // One pair of events around `reps` back-to-back launches of a kind: the
    // mean is the kernel's own time plus the dispatch gap between launches
    // (kind 8, an empty kernel, shows that gap alone).
    std::vector<hipEvent_t> ev(size_t(2) * kKinds, nullptr);
    for (auto &e : ev) Q8L_HIP(m, hipEventCreate(&e), "hipEventCreate");
    hipError_t err = hipSuccess;
    for (int k = 0; k < kKinds && err == hipSuccess; ++k) {
        rep = 0;
        if ((err = launch(k)) != hipSuccess) break;  // warm-up launch, not timed
        if ((err = hipEventRecord(ev[2 * k], s)) != hipSuccess) break;
        for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch(k);
        if (err == hipSuccess) err = hipEventRecord(ev[2 * k + 1], s);
    }
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    for (int k = 0; k < kKinds && err == hipSuccess; ++k) {
        float ms = 0.f;
        if ((err = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1])) != hipSuccess) break;
        // kind 0: not a kernel of the step; kind 3 is part of kind 2 when fused
        ms_out[k] = (k == 0 || (k == 3 && fused)) ? -1.0f : ms / float(reps);
    }
    for (auto &e : ev)
        if (e) hipEventDestroy(e);
    if (err != hipSuccess) return hip_fail(m, err, "timing decode kernels");
    return Q8L_OK;
}

q8l_status q8l_clear_kv_cache(q8l_model *m) {
    if (!m) return Q8L_E_INVALID_ARG;
    m->len = 0;
    m->kv_checked = 0;
    return Q8L_OK;
}

int32_t q8l_cache_len(const q8l_model *m) { return m ? m->len : -1; }

const char *q8l_last_error(const q8l_model *m) { return m ? m->err.c_str() : "model is NULL"; }

void q8l_destroy(q8l_model *m) {
    if (!m) return;
    for (auto &kv : m->graphs) hipGraphExecDestroy(kv.second);
    for (auto &kv : m->graph_defs) hipGraphDestroy(kv.second);
    if (m->cap) hipStreamDestroy(m->cap);
    if (m->range_host) hipHostFree(m->range_host);
    delete m;
}

// ---------------------------------------------------------------- single ops

q8l_status q8l_op_matmul_q8_0(const void *W, int64_t N, int64_t K, const float *X, int64_t T,
                              const float *norm_w, double eps, int32_t accumulate, float *Y,
                              void *stream) {
    if (!W || !X || !Y || N < 1 || K < 64 || K % 64 || T < 1 || N > (1 << 30) || K > (1 << 24) ||
        T > (1 << 20) || (reinterpret_cast<uintptr_t>(W) & 15) || (reinterpret_cast<uintptr_t>(X) & 15) ||
        (norm_w && (reinterpret_cast<uintptr_t>(norm_w) & 15)))
        return Q8L_E_INVALID_ARG;
    hipError_t e;
    if (T > kMaxTokChunk && !norm_w)
        e = launch_gemm_matmul(static_cast<const uint8_t *>(W), int(N), int(K), X, false, int(T), accumulate, Y,
                               static_cast<hipStream_t>(stream));
    else
        e = launch_matmul(static_cast<const uint8_t *>(W), int(N), int(K), X, int(T), norm_w, float(eps),
                          accumulate, Y, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8L_OK : Q8L_E_HIP;
}

q8l_status q8l_op_matmul_q5_0(const void *W, int64_t N, int64_t K, const float *X, int64_t T,
                              int32_t accumulate, float *Y, void *stream) {
    if (!W || !X || !Y || N < 1 || K < 64 || K % 64 || T < 1 || N > (1 << 30) || K > (1 << 24) ||
        T > (1 << 20) || (reinterpret_cast<uintptr_t>(W) & 15) || (reinterpret_cast<uintptr_t>(X) & 15))
        return Q8L_E_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *w = static_cast<const uint8_t *>(W);
    const hipError_t e = T > kMaxTokChunk
                             ? launch_gemm_matmul(w, int(N), int(K), X, false, int(T), accumulate, Y, s, ActScale{},
                                                  F_Q5_0)
                             : launch_matmul(w, int(N), int(K), X, int(T), nullptr, 0.f, accumulate, Y, s, F_Q5_0);
    if (e == hipErrorInvalidValue) return Q8L_E_INVALID_ARG;   // beyond the kernels' 2 GiB addressing
    return e == hipSuccess ? Q8L_OK : Q8L_E_HIP;
}

q8l_status q8l_op_matmul_kq(const void *W, int32_t dtype, int64_t N, int64_t K, const float *X, int64_t T,
                            int32_t accumulate, float *Y, void *stream) {
    if (!W || !X || !Y || (dtype != Q8L_Q4_K && dtype != Q8L_Q6_K) || N < 1 || K < kQKK || K % kQKK || T < 1 ||
        N > (1 << 30) || K > (1 << 24) || T > (1 << 20) || (reinterpret_cast<uintptr_t>(W) & 15) ||
        (reinterpret_cast<uintptr_t>(X) & 15))
        return Q8L_E_INVALID_ARG;
    const int fmt = dtype == Q8L_Q4_K ? F_Q4_K : F_Q6_K;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = T == 1 ? launch_kq_gemv(fmt, static_cast<const uint8_t *>(W), int(N), int(K), X, accumulate, Y, s)
                                : launch_gemm_kq(fmt, static_cast<const uint8_t *>(W), int(N), int(K), X, false, int(T),
                                                 accumulate, Y, s);
    if (e == hipErrorInvalidValue) return Q8L_E_INVALID_ARG;   // beyond the kernels' 2 GiB addressing
    return e == hipSuccess ? Q8L_OK : Q8L_E_HIP;
}

size_t q8l_op_attention_workspace(int32_t T, int32_t kv_len, int32_t n_head, int32_t n_head_kv,
                                  int32_t hd) {
    (void)n_head_kv;
    if (T != 1 || kv_len < 1 || n_head < 1 || hd < 8) return 256;
    const int splits = (kv_len + attn_chunk(hd) - 1) / attn_chunk(hd);
    return al256(size_t(n_head) * splits * (hd + 2) * 4);
}

q8l_status q8l_op_attention(const float *Q, const float *K, const float *V, int32_t T,
                            int32_t kv_len, int32_t kv_stride, int32_t n_head, int32_t n_head_kv,
                            int32_t hd, float *O, void *workspace, size_t workspace_bytes,
                            void *stream) {
    if (!Q || !K || !V || !O || T < 1 || kv_len < T || kv_stride < kv_len || n_head < 1 ||
        n_head_kv < 1 || n_head % n_head_kv || n_head / n_head_kv > kMaxGroup || hd % 8 || hd > 128 ||
        (reinterpret_cast<uintptr_t>(Q) & 15) || (reinterpret_cast<uintptr_t>(K) & 15) ||
        (reinterpret_cast<uintptr_t>(V) & 15))
        return Q8L_E_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (T == 1) {
        if (!workspace || workspace_bytes < q8l_op_attention_workspace(T, kv_len, n_head, n_head_kv, hd))
            return Q8L_E_INVALID_ARG;
        AttnDecodeArgs a;
        a.q = Q; a.kc = K; a.vc = V;
        a.part = static_cast<float *>(workspace);
        a.st = nullptr; a.kv_len_arg = kv_len; a.kv_stride = kv_stride;
        a.nh = n_head; a.nkv = n_head_kv; a.hd = hd;
        a.n_splits = (kv_len + attn_chunk(hd) - 1) / attn_chunk(hd);
        a.scale = 1.0f / sqrtf(float(hd));
        a.o = nullptr;
        e = launch_attn_decode(a, s);
        if (e == hipSuccess) e = launch_attn_combine(a.part, a.n_splits, kv_len, n_head, hd, O, nullptr, s);
    } else {
        AttnPrefillArgs a;
        a.q = Q; a.kc = K; a.vc = V; a.o = O; a.o_split = nullptr; a.T = T; a.kv_len = kv_len; a.kv_stride = kv_stride;
        a.nh = n_head; a.nkv = n_head_kv; a.hd = hd; a.scale = 1.0f / sqrtf(float(hd));
        e = launch_attn_prefill(a, s);
    }
    return e == hipSuccess ? Q8L_OK : Q8L_E_HIP;
}

q8l_status q8l_op_argmax(const float *x, int64_t n, uint32_t *out, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (!x || !out || n < 1 || n > (int64_t(1) << 31) || !workspace ||
        workspace_bytes < argmax_partials_bytes(n))
        return Q8L_E_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launch_argmax(x, n, out, static_cast<float *>(workspace), s) == hipSuccess ? Q8L_OK : Q8L_E_HIP;
}

}  // extern "C"
