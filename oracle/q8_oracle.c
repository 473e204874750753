/*
 * q8_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, CPU forward pass of the quantized Llama model (Q8_0 weights)
 * used to check the HIP library. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header, table
 * or constant generator with the GPU library.
 *
 * What it computes follows the pages' description of candle's quantized_llama:
 *   - "量化 llama 的一次前向", sections "forward：mask 什么时候建" (the forward:
 *     embed -> per layer norm / attention / residual / norm / MLP / residual ->
 *     final norm -> last position -> output layer; a mask only when T > 1, its
 *     first index_pos columns open and its last T columns a causal triangle),
 *     "forward_attn：自己拼 KV" (q, k, v projections, rope with index_pos, KV
 *     cache dropped when index_pos == 0, grouped heads, scale, mask, softmax),
 *     "index_pos 传错" and "换 prompt 要不要 clear_kv_cache" (the counter
 *     contract), and the 4096-row rope table bound in "from_gguf：键名写死了
 *     llama.";
 *   - "生成一个 token", section "prefill 和 decode：同一个 forward，不同的路"
 *     (score scale 1/sqrt(head_dim) before masking and softmax);
 *   - "生成一个 token", section "建模型：按名字取张量" (tensor names, the tied
 *     output layer when output.weight is absent).
 * Formulas the pages name but do not write out are taken in their textbook
 * form: RMSNorm y = x / sqrt(mean(x^2) + eps) * w; interleaved rope (pairs
 * 2j, 2j+1) with inverse frequency theta^(-2j/hd), or the NEOX pairing
 * (j, j + hd/2) with the same angles; SiLU z / (1 + e^-z).
 *
 * Precision: every weight is decoded exactly (w = f16 scale * int8, exact in
 * f64); activations, the KV cache and every sum are f64; logits are rounded
 * to f32 at the end. Rope angles follow the pages' f32 table: the angle for
 * position p and pair j is the f32 product of f32(p) and the f32-rounded
 * inverse frequency; its cos and sin are then taken in f64.
 *
 * Summation order is plain and fixed: every dot product runs k = 0..K-1.
 * OpenMP only splits independent outputs (rows, heads) across threads.
 *
 * Status codes mirror the library's boundary (same meaning, own definition).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_INVALID_ARG 1
#define ORC_E_MISSING_TENSOR 2
#define ORC_E_SHAPE 3
#define ORC_E_POS_RANGE 4
#define ORC_E_POS_MISMATCH 5
#define ORC_E_KV_FULL 6

#define ORC_QK 32        /* weights per Q8_0 block */
#define ORC_QBYTES 34    /* bytes per Q8_0 block */

typedef struct {
    int32_t n_layer, n_embd, n_head, n_head_kv, head_dim, n_ff, n_vocab, max_seq_len;
    double rms_eps, rope_theta;
    int32_t tied_output;
    int32_t rope_neox;    /* 0: pairs (2j, 2j+1) (llama); 1: pairs (j, j + hd/2) */
} orc_config;

/* Block formats of a layer's projections: Q8_0 or Q5_0 for any of them,
 * Q4_K and Q6_K for the o and down projections. */
#define ORC_FMT_Q8_0 0
#define ORC_FMT_Q4_K 1
#define ORC_FMT_Q6_K 2
#define ORC_FMT_Q5_0 3

typedef struct {
    const float *attn_norm, *ffn_norm;
    const uint8_t *wq, *wk, *wv, *wo, *wg, *wu, *wd;
    int32_t fq, fk, fv, fo, fg, fu, fd;   /* formats of the seven matrices */
} orc_layer;

typedef struct {
    orc_config c;
    const uint8_t *tok_embd;
    orc_layer *layers;
    const float *out_norm;
    const uint8_t *out;     /* == tok_embd when tied */
    double *kc, *vc;        /* [L][nkv][max_seq][hd] */
    int32_t len;            /* positions held in the cache */
    int64_t n_matmul, n_rmsnorm, n_rope;  /* calls in the last forward */
} orc_model;

/* ---- scalar pieces ---------------------------------------------------- */

/* IEEE binary16 -> f64, including subnormals (value = m * 2^-24 when e == 0). */
double orc_f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

/* Decode one row of K weights (K/32 blocks of 34 bytes) into f64. */
/* Two other 32-weight block formats of the same file family (the public GGUF
 * block definitions; the pages fix only their sizes, "速度", section "CPU GGUF"):
 * Q4_0 = f16 d + 16 bytes: weight i < 16 is the low nibble of byte i, weight
 * i + 16 its high nibble, value = d * (nibble - 8). Q5_0 = f16 d + a 32-bit
 * little-endian word of fifth bits (bit i for weight i) + 16 bytes of nibbles
 * in the Q4_0 order, value = d * ((nibble | fifth bit << 4) - 16). */
void orc_dequant_q4_0_row(const uint8_t *row, int64_t K, double *out) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const uint8_t *blk = row + b * 18;
        double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int i = 0; i < 16; ++i) {
            out[b * 32 + i] = d * (double)((blk[2 + i] & 0x0f) - 8);
            out[b * 32 + i + 16] = d * (double)((blk[2 + i] >> 4) - 8);
        }
    }
}

void orc_dequant_q5_0_row(const uint8_t *row, int64_t K, double *out) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const uint8_t *blk = row + b * 22;
        double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
        for (int i = 0; i < 16; ++i) {
            int lo = (blk[6 + i] & 0x0f) | (int)(((qh >> i) & 1u) << 4);
            int hi = (blk[6 + i] >> 4) | (int)(((qh >> (i + 16)) & 1u) << 4);
            out[b * 32 + i] = d * (double)(lo - 16);
            out[b * 32 + i + 16] = d * (double)(hi - 16);
        }
    }
}

/* Two 256-weight "K" formats (public GGUF block definitions; the pages fix
 * their sizes through the Q4_K_M table of "速度", section "CPU GGUF").
 * Q4_K, 144 bytes: f16 d, f16 dmin, 12 bytes holding eight 6-bit scales and
 * eight 6-bit mins, 128 bytes of nibbles. Sub-block j (32 weights) has scale s_j
 * and min m_j; for j < 4 they are the low 6 bits of bytes j and j + 4; for
 * j >= 4 the scale is the low nibble of byte j + 4 with the top two bits of
 * byte j - 4 above it, the min the high nibble of byte j + 4 with the top two
 * bits of byte j above it. Weight l of sub-block j = d*s_j*q - dmin*m_j, q the
 * low (j even) or high (j odd) nibble of byte 32*(j/2) + l. */
static void q4k_scale_min(int j, const uint8_t *sc, int *s, int *m) {
    if (j < 4) {
        *s = sc[j] & 63;
        *m = sc[j + 4] & 63;
    } else {
        *s = (sc[j + 4] & 0x0f) | ((sc[j - 4] >> 6) << 4);
        *m = (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4);
    }
}

void orc_dequant_q4_k_row(const uint8_t *row, int64_t K, double *out) {
    for (int64_t b = 0; b < K / 256; ++b) {
        const uint8_t *blk = row + b * 144;
        const double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        const double dmin = orc_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
        const uint8_t *sc = blk + 4, *qs = blk + 16;
        for (int j = 0; j < 8; ++j) {
            int s, m;
            q4k_scale_min(j, sc, &s, &m);
            for (int l = 0; l < 32; ++l) {
                const uint8_t byte = qs[32 * (j / 2) + l];
                const int q = (j & 1) ? (byte >> 4) : (byte & 0x0f);
                out[b * 256 + 32 * j + l] = d * (double)s * (double)q - dmin * (double)m;
            }
        }
    }
}

/* Q6_K, 210 bytes: 128 bytes of low nibbles, 64 bytes of 2-bit high parts,
 * 16 int8 scales (one per 16 weights), f16 d. In each half (128 weights: low
 * nibbles 64h.., high parts 32h.., scales 8h..), weight 32*k + l (k = 0..3,
 * l = 0..31) takes the low (k < 2) or high (k >= 2) nibble of low byte
 * l + 32*(k odd), the 2-bit field k of high byte l, minus 32, times d and
 * scale 2*k + l/16. */
void orc_dequant_q6_k_row(const uint8_t *row, int64_t K, double *out) {
    for (int64_t b = 0; b < K / 256; ++b) {
        const uint8_t *blk = row + b * 210;
        const uint8_t *ql = blk, *qh = blk + 128;
        const int8_t *sc = (const int8_t *)(blk + 192);
        const double d = orc_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
        for (int h = 0; h < 2; ++h)
            for (int k = 0; k < 4; ++k)
                for (int l = 0; l < 32; ++l) {
                    const uint8_t lo = ql[64 * h + l + 32 * (k & 1)];
                    const int nib = (k < 2) ? (lo & 0x0f) : (lo >> 4);
                    const int q = (nib | (((qh[32 * h + l] >> (2 * k)) & 3) << 4)) - 32;
                    out[b * 256 + 128 * h + 32 * k + l] = d * (double)sc[8 * h + 2 * k + l / 16] * (double)q;
                }
    }
}

void orc_dequant_row(const uint8_t *row, int64_t K, double *out) {
    for (int64_t b = 0; b < K / ORC_QK; ++b) {
        const uint8_t *blk = row + b * ORC_QBYTES;
        double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int i = 0; i < ORC_QK; ++i) out[b * ORC_QK + i] = d * (double)(int8_t)blk[2 + i];
    }
}

static int64_t row_bytes(int64_t K) { return K / ORC_QK * ORC_QBYTES; }

static int64_t fmt_row_bytes(int32_t fmt, int64_t K) {
    return fmt == ORC_FMT_Q4_K ? K / 256 * 144 : fmt == ORC_FMT_Q6_K ? K / 256 * 210
         : fmt == ORC_FMT_Q5_0 ? K / 32 * 22 : row_bytes(K);
}

static void dequant_fmt(int32_t fmt, const uint8_t *row, int64_t K, double *out) {
    if (fmt == ORC_FMT_Q4_K) orc_dequant_q4_k_row(row, K, out);
    else if (fmt == ORC_FMT_Q6_K) orc_dequant_q6_k_row(row, K, out);
    else if (fmt == ORC_FMT_Q5_0) orc_dequant_q5_0_row(row, K, out);
    else orc_dequant_row(row, K, out);
}

/* Y[t][n] = sum_k W[n][k] * X[t][k] for T input rows; W is Q8_0 [N][K]. */
/* Y[t] = W X[t] for a matrix in block format fmt. */
void orc_matmul_fmt(const uint8_t *W, int32_t fmt, int64_t N, int64_t K, const double *X, int64_t T,
                    double *Y) {
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            dequant_fmt(fmt, W + n * fmt_row_bytes(fmt, K), K, w);
            for (int64_t t = 0; t < T; ++t) {
                const double *x = X + t * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += w[k] * x[k];
                Y[t * N + n] = acc;
            }
        }
        free(w);
    }
}

void orc_matmul_q8(const uint8_t *W, int64_t N, int64_t K, const double *X, int64_t T,
                   double *Y) {
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            orc_dequant_row(W + n * row_bytes(K), K, w);
            for (int64_t t = 0; t < T; ++t) {
                const double *x = X + t * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += w[k] * x[k];
                Y[t * N + n] = acc;
            }
        }
        free(w);
    }
}

/* y = x / sqrt(mean(x^2) + eps) * w, one row of H. */
void orc_rmsnorm(const double *x, const float *w, int64_t H, double eps, double *y) {
    double ss = 0.0;
    for (int64_t k = 0; k < H; ++k) ss += x[k] * x[k];
    double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t k = 0; k < H; ++k) y[k] = x[k] * r * (double)w[k];
}

/* The rope angle of pair j at position p, as the pages' f32 table holds it. */
double orc_rope_angle(int64_t p, int64_t j, int64_t hd, double theta) {
    float inv_freq = (float)pow(theta, -2.0 * (double)j / (double)hd);
    float ang = (float)p * inv_freq;
    return (double)ang;
}

/* Rotate one head vector (hd values) in place: pairs (2j, 2j+1). */
void orc_rope_i(double *v, int64_t hd, int64_t p, double theta) {
    for (int64_t j = 0; j < hd / 2; ++j) {
        double a = orc_rope_angle(p, j, hd, theta);
        double c = cos(a), s = sin(a);
        double x0 = v[2 * j], x1 = v[2 * j + 1];
        v[2 * j] = x0 * c - x1 * s;
        v[2 * j + 1] = x0 * s + x1 * c;
    }
}

/* The other convention ("量化 llama 的一次前向", section "RoPE：两种约定，按架构名选":
 * the NEOX one, dimension j paired with dimension j + hd/2), same angles. */
void orc_rope_neox(double *v, int64_t hd, int64_t p, double theta) {
    const int64_t half = hd / 2;
    for (int64_t j = 0; j < half; ++j) {
        double a = orc_rope_angle(p, j, hd, theta);
        double c = cos(a), s = sin(a);
        double x0 = v[j], x1 = v[j + half];
        v[j] = x0 * c - x1 * s;
        v[j + half] = x0 * s + x1 * c;
    }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Attention for one query vector q (hd) over n_keys keys K[j], values V[j]
 * (row stride hd): scores q.k_j / sqrt(hd); keys with j > last_visible get
 * -inf (pass last_visible >= n_keys - 1 for no mask); softmax; weighted sum.
 */
void orc_attend(const double *q, const double *K, const double *V, int64_t n_keys,
                int64_t hd, int64_t last_visible, double *o) {
    double *s = (double *)malloc(sizeof(double) * (n_keys > 0 ? n_keys : 1));
    double scale = 1.0 / sqrt((double)hd);
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < hd; ++d) dot += q[d] * K[j * hd + d];
        s[j] = (j > last_visible) ? -INFINITY : dot * scale;
        if (s[j] > m) m = s[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        z += s[j];
    }
    for (int64_t d = 0; d < hd; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        double pj = s[j] / z;
        for (int64_t d = 0; d < hd; ++d) o[d] += pj * V[j * hd + d];
    }
    free(s);
}

/* ---- model ------------------------------------------------------------- */

static int cfg_ok(const orc_config *c) {
    if (c->n_layer < 1 || c->n_embd < 1 || c->n_head < 1 || c->n_head_kv < 1 ||
        c->head_dim < 2 || c->n_ff < 1 || c->n_vocab < 1 || c->max_seq_len < 1)
        return 0;
    if (c->n_head % c->n_head_kv || c->head_dim % 2) return 0;
    if (c->n_embd % ORC_QK || c->n_ff % ORC_QK || (c->n_head * c->head_dim) % ORC_QK) return 0;
    return 1;
}

/*
 * tensors: pointers in canonical order -- token_embd; per layer attn_norm,
 * attn_q, attn_k, attn_v, attn_output, ffn_norm, ffn_gate, ffn_up, ffn_down;
 * output_norm; output (only when not tied). The model borrows them.
 */
orc_model *orc_create_fmt7(const orc_config *c, const void *const *tensors, const int32_t *fmts);

orc_model *orc_create(const orc_config *c, const void *const *tensors) {
    return orc_create_fmt7(c, tensors, NULL);
}

/* As orc_create, with per-layer block formats of attn_output and ffn_down
 * (ORC_FMT_*; NULL = Q8_0 everywhere; the other matrices Q8_0). */
orc_model *orc_create_fmt(const orc_config *c, const void *const *tensors, const int32_t *wo_fmt,
                          const int32_t *wd_fmt) {
    if (!c || c->n_layer < 1) return NULL;
    int32_t *f = (int32_t *)calloc((size_t)c->n_layer * 7, sizeof(int32_t));
    for (int l = 0; l < c->n_layer; ++l) {
        f[7 * l + 3] = wo_fmt ? wo_fmt[l] : ORC_FMT_Q8_0;
        f[7 * l + 6] = wd_fmt ? wd_fmt[l] : ORC_FMT_Q8_0;
    }
    orc_model *m = orc_create_fmt7(c, tensors, f);
    free(f);
    return m;
}

/* As orc_create, with the block format of every matrix: fmts[7*l + i] for
 * layer l and i = q, k, v, o, gate, up, down (ORC_FMT_*; NULL = Q8_0
 * everywhere). Q4_K / Q6_K only for o and down, with whole 256-weight blocks
 * per row. */
orc_model *orc_create_fmt7(const orc_config *c, const void *const *tensors, const int32_t *fmts) {
    if (!c || !tensors || !cfg_ok(c)) return NULL;
    for (int l = 0; l < c->n_layer && fmts; ++l)
        for (int i = 0; i < 7; ++i) {
            const int32_t f = fmts[7 * l + i];
            const int64_t K = i == 3 ? (int64_t)c->n_head * c->head_dim : i == 6 ? c->n_ff : c->n_embd;
            if (f < 0 || f > 3) return NULL;
            if ((f == ORC_FMT_Q4_K || f == ORC_FMT_Q6_K) && ((i != 3 && i != 6) || K % 256)) return NULL;
        }
    orc_model *m = (orc_model *)calloc(1, sizeof(orc_model));
    m->c = *c;
    int64_t i = 0;
    m->tok_embd = (const uint8_t *)tensors[i++];
    m->layers = (orc_layer *)calloc((size_t)c->n_layer, sizeof(orc_layer));
    for (int l = 0; l < c->n_layer; ++l) {
        orc_layer *L = &m->layers[l];
        L->attn_norm = (const float *)tensors[i++];
        L->wq = (const uint8_t *)tensors[i++];
        L->wk = (const uint8_t *)tensors[i++];
        L->wv = (const uint8_t *)tensors[i++];
        L->wo = (const uint8_t *)tensors[i++];
        L->ffn_norm = (const float *)tensors[i++];
        L->wg = (const uint8_t *)tensors[i++];
        L->wu = (const uint8_t *)tensors[i++];
        L->wd = (const uint8_t *)tensors[i++];
        const int32_t *f = fmts ? fmts + 7 * l : NULL;
        L->fq = f ? f[0] : ORC_FMT_Q8_0;
        L->fk = f ? f[1] : ORC_FMT_Q8_0;
        L->fv = f ? f[2] : ORC_FMT_Q8_0;
        L->fo = f ? f[3] : ORC_FMT_Q8_0;
        L->fg = f ? f[4] : ORC_FMT_Q8_0;
        L->fu = f ? f[5] : ORC_FMT_Q8_0;
        L->fd = f ? f[6] : ORC_FMT_Q8_0;
    }
    m->out_norm = (const float *)tensors[i++];
    m->out = c->tied_output ? m->tok_embd : (const uint8_t *)tensors[i++];
    size_t kv = (size_t)c->n_layer * c->n_head_kv * c->max_seq_len * c->head_dim;
    m->kc = (double *)calloc(kv, sizeof(double));
    m->vc = (double *)calloc(kv, sizeof(double));
    if (!m->kc || !m->vc) {
        free(m->kc); free(m->vc); free(m->layers); free(m);
        return NULL;
    }
    m->len = 0;
    return m;
}

void orc_destroy(orc_model *m) {
    if (!m) return;
    free(m->kc); free(m->vc); free(m->layers); free(m);
}

void orc_clear_kv_cache(orc_model *m) { m->len = 0; }
int32_t orc_cache_len(const orc_model *m) { return m->len; }
void orc_counts(const orc_model *m, int64_t *out3) {
    out3[0] = m->n_matmul; out3[1] = m->n_rmsnorm; out3[2] = m->n_rope;
}

static double *kslot(orc_model *m, double *base, int l, int g, int64_t pos) {
    const orc_config *c = &m->c;
    return base + (((size_t)l * c->n_head_kv + g) * c->max_seq_len + pos) * c->head_dim;
}

/*
 * forward(tokens[0..T), index_pos) -> logits of the last position.
 * Checks, in order, before anything changes:
 *   1. T >= 1, every token < V, index_pos >= 0           else E_INVALID_ARG
 *   2. index_pos + T <= max_seq_len                      else E_POS_RANGE
 *   3. index_pos == 0 drops the cache (len := 0)
 *   4. T > 1 requires index_pos == len                   else E_POS_MISMATCH
 *      (T == 1 is not checked: rope uses index_pos, the new entry goes to
 *      slot len, and the single query sees every cached key)
 *   5. len + T <= max_seq_len                            else E_KV_FULL
 * logits64 (optional) receives the f64 values before rounding.
 */
int orc_forward(orc_model *m, const uint32_t *tokens, int32_t T, int32_t index_pos,
                float *logits, double *logits64) {
    const orc_config *c = &m->c;
    if (T < 1 || index_pos < 0) return ORC_E_INVALID_ARG;
    for (int32_t i = 0; i < T; ++i)
        if (tokens[i] >= (uint32_t)c->n_vocab) return ORC_E_INVALID_ARG;
    if ((int64_t)index_pos + T > c->max_seq_len) return ORC_E_POS_RANGE;
    int32_t len = (index_pos == 0) ? 0 : m->len;
    if (T > 1 && index_pos != len) return ORC_E_POS_MISMATCH;
    if ((int64_t)len + T > c->max_seq_len) return ORC_E_KV_FULL;

    const int64_t H = c->n_embd, nh = c->n_head, nkv = c->n_head_kv, hd = c->head_dim;
    const int64_t F = c->n_ff, V = c->n_vocab, QD = nh * hd, KVD = nkv * hd;
    const int64_t group = nh / nkv;
    const int64_t kv_len = (int64_t)len + T;

    double *x = (double *)malloc(sizeof(double) * T * H);
    double *u = (double *)malloc(sizeof(double) * T * H);
    double *q = (double *)malloc(sizeof(double) * T * QD);
    double *k = (double *)malloc(sizeof(double) * T * KVD);
    double *v = (double *)malloc(sizeof(double) * T * KVD);
    double *att = (double *)malloc(sizeof(double) * T * QD);
    double *y = (double *)malloc(sizeof(double) * T * (H > F ? H : F));
    double *g = (double *)malloc(sizeof(double) * T * F);
    double *up = (double *)malloc(sizeof(double) * T * F);
    m->n_matmul = m->n_rmsnorm = m->n_rope = 0;

    /* embedding: x_i = dequant(E[t_i]) */
    for (int32_t i = 0; i < T; ++i)
        orc_dequant_row(m->tok_embd + (int64_t)tokens[i] * row_bytes(H), H, x + i * H);

    for (int l = 0; l < c->n_layer; ++l) {
        const orc_layer *L = &m->layers[l];
        /* attention block */
        for (int32_t i = 0; i < T; ++i) orc_rmsnorm(x + i * H, L->attn_norm, H, c->rms_eps, u + i * H);
        m->n_rmsnorm++;
        orc_matmul_fmt(L->wq, L->fq, QD, H, u, T, q);
        orc_matmul_fmt(L->wk, L->fk, KVD, H, u, T, k);
        orc_matmul_fmt(L->wv, L->fv, KVD, H, u, T, v);
        m->n_matmul += 3;
        for (int32_t i = 0; i < T; ++i) {
            void (*rope)(double *, int64_t, int64_t, double) = c->rope_neox ? orc_rope_neox : orc_rope_i;
            for (int64_t h = 0; h < nh; ++h) rope(q + i * QD + h * hd, hd, (int64_t)index_pos + i, c->rope_theta);
            for (int64_t h = 0; h < nkv; ++h) rope(k + i * KVD + h * hd, hd, (int64_t)index_pos + i, c->rope_theta);
        }
        m->n_rope += 2;
        for (int32_t i = 0; i < T; ++i)
            for (int64_t h = 0; h < nkv; ++h) {
                memcpy(kslot(m, m->kc, l, (int)h, len + i), k + i * KVD + h * hd, sizeof(double) * hd);
                memcpy(kslot(m, m->vc, l, (int)h, len + i), v + i * KVD + h * hd, sizeof(double) * hd);
            }
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t h = 0; h < nh; ++h)
            for (int32_t i = 0; i < T; ++i) {
                int64_t gh = h / group;   /* query head h reads KV head h / (nh/nkv) */
                /* mask iff T > 1: query i sees keys j <= index_pos + i */
                int64_t last = (T > 1) ? (int64_t)index_pos + i : kv_len - 1;
                orc_attend(q + i * QD + h * hd, kslot(m, m->kc, l, (int)gh, 0),
                           kslot(m, m->vc, l, (int)gh, 0), kv_len, hd, last, att + i * QD + h * hd);
            }
        orc_matmul_fmt(L->wo, L->fo, H, QD, att, T, y);
        m->n_matmul += 1;
        for (int64_t e = 0; e < T * H; ++e) x[e] += y[e];

        /* MLP block */
        for (int32_t i = 0; i < T; ++i) orc_rmsnorm(x + i * H, L->ffn_norm, H, c->rms_eps, u + i * H);
        m->n_rmsnorm++;
        orc_matmul_fmt(L->wg, L->fg, F, H, u, T, g);
        orc_matmul_fmt(L->wu, L->fu, F, H, u, T, up);
        for (int64_t e = 0; e < T * F; ++e) g[e] = orc_silu(g[e]) * up[e];
        orc_matmul_fmt(L->wd, L->fd, H, F, g, T, y);
        m->n_matmul += 3;
        for (int64_t e = 0; e < T * H; ++e) x[e] += y[e];
    }

    /* final norm on the last position only, then the output layer */
    orc_rmsnorm(x + (int64_t)(T - 1) * H, m->out_norm, H, c->rms_eps, u);
    m->n_rmsnorm++;
    double *lg = (double *)malloc(sizeof(double) * V);
    orc_matmul_q8(m->out, V, H, u, 1, lg);
    m->n_matmul += 1;
    for (int64_t n = 0; n < V; ++n) {
        if (logits) logits[n] = (float)lg[n];
        if (logits64) logits64[n] = lg[n];
    }
    m->len = (int32_t)kv_len;

    free(lg); free(x); free(u); free(q); free(k); free(v); free(att); free(y); free(g); free(up);
    return ORC_OK;
}

/* Greedy pick: index of the largest value, the lowest index on ties. */
int64_t orc_argmax(const float *v, int64_t n) {
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i)
        if (v[i] > v[best]) best = i;
    return best;
}

/* Read back one cached key or value vector (for tests). kind 0 = K, 1 = V. */
int orc_read_cache(orc_model *m, int kind, int l, int g, int64_t pos, double *out) {
    const orc_config *c = &m->c;
    if (l < 0 || l >= c->n_layer || g < 0 || g >= c->n_head_kv || pos < 0 || pos >= c->max_seq_len)
        return ORC_E_INVALID_ARG;
    memcpy(out, kslot(m, kind ? m->vc : m->kc, l, g, pos), sizeof(double) * c->head_dim);
    return ORC_OK;
}
