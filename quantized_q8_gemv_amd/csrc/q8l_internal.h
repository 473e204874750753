// q8l_internal.h -- structures shared by the host runtime and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8l {

constexpr int kThreads = 256;        // every kernel runs 256-thread workgroups (4 wave64)
constexpr int kQK = 32;              // weights per Q8_0 block
constexpr int kQBytes = 34;          // bytes per Q8_0 block
constexpr int kPairBytes = 68;       // two blocks: the unit a lane decodes (4-byte aligned)
constexpr int kPairWeights = 64;
constexpr int kMaxTokChunk = 16;     // tokens per workgroup in the multi-token GEMV
constexpr int kGemmMinTokens = 6;    // forward calls with at least this many tokens use the MFMA GEMM
constexpr int kInlineTokens = 256;   // token ids passed in kernel arguments per launch
constexpr int kAttnChunk = 64;       // keys per split in decode attention
constexpr int kMaxGroup = 16;        // query heads per KV head supported in-kernel

// Per-call step state, in device memory. Graph-replayed kernels read it
// instead of kernel arguments, so one captured decode graph serves every step.
struct StepState {
    int32_t pos;        // rope position of token 0 (index_pos)
    int32_t slot;       // KV slot of token 0 (positions cached before the call)
    int32_t T;          // tokens in the call
    int32_t step;       // generation step counter
    uint32_t token;     // single-token input (decode)
    int32_t advance;    // 1: after the argmax, token := argmax, pos++, slot++, step++
    float *logits_out;  // lm_head destination
    uint32_t *argmax_out;  // optional argmax destination
    uint32_t *ids_out;     // generation: ids_out[step] := argmax
};

struct SetStateArgs {
    int32_t pos, slot, T, step;
    int32_t advance;
    int32_t tok_offset, tok_count;   // tokens written to tok_buf[tok_offset ..)
    int32_t set_header;              // 0: only copy tokens
    float *logits_out;
    uint32_t *argmax_out;
    uint32_t *ids_out;
    uint32_t tokens[kInlineTokens];
};

// How a GEMV walks one weight matrix: K = P pairs of blocks per row, taken in
// chunks of PC pairs; a workgroup owns NR rows.
struct GemvShape {
    int K;        // weights per row
    int P;        // 64-weight pairs per row
    int PC;       // pairs per K-chunk (divides P)
    int NR;       // rows per workgroup (NR * PC <= 256)
    int rowbytes; // P * pb
    int pb;       // bytes per 64-weight pair: 68 (Q8_0) or 44 (Q5_0)
};

// Split-K partial sums waiting to be added to the residual row: the kernels
// with a norm in front read x + (p_0 + p_1 + ... + p_{n-1}) (each p_i a row of
// `stride` floats at part + i * stride, summed in index order) and workgroup
// 0 writes that row to xout, the residual for what follows.
struct PartSrc {
    const float *part = nullptr;
    int n = 0;
    int stride = 0;
    float *xout = nullptr;
};

// ---- launchers (k_*.hip) -------------------------------------------------

// Block formats a matrix may be stored in. Q4_K and Q6_K (256-weight blocks)
// are accepted for the plain-matmul roles (o and down projections).
// Q5_0 (32-weight blocks: f16 d, a 32-bit word of fifth bits, 16 bytes of
// nibbles; weight = d * ((nibble | bit << 4) - 16)) is accepted for the q, k,
// v, o, gate and up projections.
enum WFmt { F_Q8_0 = 0, F_Q4_K = 1, F_Q6_K = 2, F_Q5_0 = 3 };
constexpr int kQ5Bytes = 22;         // bytes per Q5_0 block
constexpr int kQ5PairBytes = 44;     // two Q5_0 blocks: 64 weights
constexpr int kQKK = 256;            // weights per Q4_K / Q6_K block
constexpr int kQ4KBytes = 144;       // f16 d, f16 dmin, 12 scale/min bytes, 128 nibble bytes
constexpr int kQ6KBytes = 210;       // 128 low-nibble bytes, 64 high-bit bytes, 16 int8 scales, f16 d

// Block formats a GEMV kernel instance decodes: each kernel is built once
// per mode, so the Q8_0 instances carry no Q5_0 decoding (its registers would
// lower their occupancy). PM_MIXED picks per matrix at run time (q, k and v
// of one layer in different formats).
enum PairMode { PM_Q8 = 0, PM_Q5 = 1, PM_MIXED = 2 };
inline int pair_mode(int f0, int f1, int f2) {
    if (f0 == f1 && f1 == f2) return f0 == F_Q5_0 ? PM_Q5 : PM_Q8;
    return PM_MIXED;
}

// 256-weight block formats: the K-format GEMV and GEMM kernels.
__host__ __device__ inline bool kq_format(int fmt) { return fmt == F_Q4_K || fmt == F_Q6_K; }

__host__ __device__ inline int64_t fmt_row_bytes(int fmt, int64_t K) {
    return fmt == F_Q4_K ? K / kQKK * kQ4KBytes
         : fmt == F_Q6_K ? K / kQKK * kQ6KBytes
         : fmt == F_Q5_0 ? K / kQK * kQ5Bytes
                         : K / kQK * kQBytes;
}

struct LayerPtrs {
    const uint8_t *wq, *wk, *wv, *wo, *wg, *wu, *wd;
    const float *attn_norm, *ffn_norm;
    int fq, fk, fv, fo, fg, fu, fd;  // WFmt of each matrix
};

struct Dims {
    int H, nh, nkv, hd, F, V, max_seq;
    float eps;
    int rope_neox;  // 1: pairs (j, j + hd/2), applied by launch_rope_neox after q/k/v
};

hipError_t launch_set_state(const SetStateArgs &a, StepState *st, uint32_t *tok_buf,
                            hipStream_t s);
hipError_t launch_rope_table(float2 *table, int max_seq, int hd, double theta, hipStream_t s);
hipError_t launch_noop(hipStream_t s);
// NEOX rotation of the T new tokens' q (rows of [T][nh*hd]) and k (cache slots
// st->slot + t) at positions st->pos + t.
hipError_t launch_rope_neox(const Dims &d, const StepState *st, const float2 *rope, float *q, float *kc,
                            int T, hipStream_t s, uint32_t *range_flag = nullptr);
// Sets *range_flag when a value of positions [lo, hi) of any layer's K or V
// cache is outside the f16 pairs' range (before a prefill reads positions a
// decode step wrote).
hipError_t launch_kv_range(const float *kc, const float *vc, size_t layer_stride, int n_layer, int nkv, int max_seq,
                           int hd, int lo, int hi, uint32_t *range_flag, hipStream_t s);
hipError_t launch_embed(const uint8_t *E, int H, int V, const StepState *st,
                        const uint32_t *tok_buf, int T, int from_state_token, float *x,
                        hipStream_t s);

// q/k/v projections with RMSNorm in front, rope on q and k, k/v written to
// the cache at slot+t. Tokens [0, T) in chunks of up to kMaxTokChunk.
// With embed (decode only, T = 1): the input row is the embedding of the
// step's token (Q8_0 rows of embed), and xres receives it as the residual.
hipError_t launch_qkv(const Dims &d, const LayerPtrs &w, const float *x, const StepState *st,
                      const float2 *rope, float *q, float *kc, float *vc, int T,
                      hipStream_t s, const uint8_t *embed = nullptr, float *xres = nullptr,
                      const PartSrc &ps = PartSrc{}, uint32_t *range_flag = nullptr);
// Single-token products for short rows (K = 64 P, P in a fixed set of small
// values: wgemv_fits): one wave per row pair, no LDS or barriers
// (k_wgemv.hip). launch_qkv, launch_gateup and launch_matmul (without a norm)
// take this path by themselves when T == 1 and the rows fit.
bool wgemv_fits(int K);
hipError_t launch_wqkv(const Dims &d, const LayerPtrs &w, const float *x, const StepState *st, const float2 *rope,
                       float *q, float *kc, float *vc, hipStream_t s, const uint8_t *embed, float *xres,
                       const PartSrc &ps);
hipError_t launch_wgateup(const Dims &d, const LayerPtrs &w, const float *x, float *h, hipStream_t s,
                          const PartSrc &ps);
hipError_t launch_wmatmul(const uint8_t *W, int N, int K, const float *x, int accumulate, float *y, hipStream_t s,
                          int fmt = F_Q8_0);
// Single-token products of rows of kXMinPairs .. 64 pairs with the
// activations in registers (k_xgemv.hip; PartSrc not taken: callers use the
// LDS kernels when partial sums are pending). xgemv_slices: 1 for such rows,
// 2 or 4 for rows of up to 128 or 256 pairs (the plain product only), 0
// otherwise. launch_xlmhead writes n_partials argmax partials. Each returns
// hipErrorNotSupported, launching nothing, for shapes or formats it does not
// take (the caller then uses the LDS kernels).
constexpr int kXMinPairs = 32;
bool xgemv_fits(int K);
int xgemv_slices(int K);
hipError_t launch_xmatmul(const uint8_t *W, int N, int K, const float *x, int accumulate, float *y, hipStream_t s,
                          int fmt);
hipError_t launch_xgateup(const Dims &dm, const LayerPtrs &w, const float *x, float *h, hipStream_t s);
// Grid of the output layer for rows under kXMinPairs pairs (several rows per
// wave; also its partials count); 0 when such rows do not fit it.
int xlmhead_short_blocks(int V, int K);
hipError_t launch_xlmhead(const Dims &dm, const uint8_t *Wout, const float *out_norm, const float *x_last,
                          StepState *st, float *partials, int n_partials, hipStream_t s);
// Y[t] (+)= W U[t] for generic use (o-proj / down with accumulate = 1).
// fmt: Q8_0 or Q5_0.
hipError_t launch_matmul(const uint8_t *W, int N, int K, const float *X, int T,
                         const float *norm_w, float eps, int accumulate, float *Y,
                         hipStream_t s, int fmt = F_Q8_0);
// Decode o-projection after an attention of 2..kMergeMaxSplits splits: the
// merge of the split partials (part, [nh][n_splits][hd + 2]) is the GEMV's
// prologue (no merge kernel); Y += W o. Every workgroup of the GEMV reads all
// partials, so this pays only while they are few: oproj_merges says when
// (at most kMergeMaxBytes of partials; measured: the 135M shape, 9 heads of
// 64, merges up to 8 splits 6-9 % faster per token; the 7B-class shape, 32
// heads of 128, was 2-5 % slower with 4 or 8 splits).
constexpr int kMergeMaxSplits = 8;
constexpr int kMergeMaxBytes = 24 * 1024;
inline bool oproj_merges(const Dims &d, int n_splits) {
    return n_splits > 1 && n_splits <= kMergeMaxSplits &&
           int64_t(d.nh) * n_splits * (d.hd + 2) * 4 <= kMergeMaxBytes;
}
hipError_t launch_oproj_merged(const uint8_t *W, int N, int K, const float *part, int n_splits, int hd,
                               const StepState *st, float *Y, hipStream_t s);
// h[t] = silu(Wg u[t]) * (Wu u[t]), u = rmsnorm(x[t]).
hipError_t launch_gateup(const Dims &d, const LayerPtrs &w, const float *x, float *h, int T,
                         hipStream_t s, const PartSrc &ps = PartSrc{});
// logits = Wout rmsnorm(x[T-1]); argmax by the last workgroup; state update.
// Output layer logits + per-workgroup argmax partials; then the one-workgroup
// merge (which also advances the step state for on-device generation).
hipError_t launch_lmhead(const Dims &d, const uint8_t *Wout, const float *out_norm,
                         const float *x_last, StepState *st, float *partials, hipStream_t s,
                         const PartSrc &ps = PartSrc{});
hipError_t launch_argmax_finish(const Dims &d, const float *partials, StepState *st,
                                hipStream_t s);
hipError_t launch_argmax(const float *x, int64_t n, uint32_t *out, float *partials,
                         hipStream_t s);
size_t argmax_partials_bytes(int64_t n);

// Decode attention (one query per head over kv_len keys, no mask).
struct AttnDecodeArgs {
    const float *q;      // [nh][hd]
    const float *kc, *vc; // [nkv][kv_stride][hd]
    float *part;         // [nh][n_splits][hd + 2]
    const StepState *st; // kv_len = st->slot + 1 when kv_len_arg < 0
    int kv_len_arg;
    int kv_stride, nh, nkv, hd;
    int n_splits;        // workgroups per KV group launched
    float scale;
    float *o;            // n_splits == 1 only: the normalised output [nh][hd] instead of partials (or NULL)
};
hipError_t launch_attn_decode(const AttnDecodeArgs &a, hipStream_t s);
// Decode attention of a cache that fits one split (kv_len <= attn_chunk(hd))
// fused with the o-projection, split over KV groups: part[g][n] = the sum over
// group g's columns of W_o[n][.] times its heads' normalised output; the
// residual add of sum_g part[g] is left to the next kernel with a norm in
// front (PartSrc). W_o Q8_0 [N][nh*hd]; part [nkv][N].
struct AttnODecodeArgs {
    AttnDecodeArgs at;
    const uint8_t *wo;
    int N;          // rows of W_o (the model width)
    int rows;       // rows of W_o per workgroup
    float *part;
};
constexpr int kOPad = 68;      // floats per staged 64-value output pair (bank padding)
constexpr int kAttnOWgs = 64;  // workgroups the fused attention + o-projection aims for
constexpr size_t kFuseAttnOMaxBytes = 16 * 1024;  // largest n_head_kv * width * 4 fused
bool attn_o_fits(const Dims &d);  // whole 64-column pairs per group, at most kThreads per row
int attn_o_rows(const Dims &d);
hipError_t launch_attn_o(const AttnDecodeArgs &a, const uint8_t *wo, int N, float *part, hipStream_t s,
                         int fmt = F_Q8_0);

// Merge split partials into o; with st set, kv_len is read from st->slot + 1.
hipError_t launch_attn_combine(const float *part, int n_splits, int kv_len, int nh, int hd,
                               float *o, const StepState *st, hipStream_t s);
int attn_decode_splits(int kv_len, int hd);
// Keys per decode attention split.
__host__ __device__ inline int attn_chunk(int hd) { return hd <= 64 ? 64 : 32; }
// LDS of one decode attention split: q (G*hd), K tile (chunk*(hd+kKPad)),
// V tile (chunk*hd), one row of chunk softmax numerators per wave, in floats.
constexpr int kKPad = 4;
__host__ __device__ inline size_t attn_decode_lds(int G, int hd) {
    const int C = attn_chunk(hd);
    return sizeof(float) * (size_t(G) * hd + size_t(C) * (hd + kKPad) + size_t(C) * hd + size_t(kThreads / 64) * C);
}
// The fused attention + o-projection stages the group's output after that,
// at a 16-byte boundary (it is read as float4).
__host__ __device__ inline size_t attn_o_xs_offset(int G, int hd) { return (attn_decode_lds(G, hd) + 15) & ~size_t(15); }
size_t lmhead_partials_bytes(int V, int K);

// Scaling of the activations the MFMA kernels take as f16 pairs (hi + lo):
//   rs        per-token factor of a normalised input: the rows of u were
//             multiplied by 1/rs[t] (a power of two putting the row's largest
//             |u| in [2^14, 2^15)); the epilogue multiplies by rs[t]
//   eg, el    per-token and per-(token, 32-wide block) exponents of split
//             planes written by another kernel (el[t][b]: block b was
//             multiplied by 2^el[t][b], 0 unless a value would reach 2^15;
//             eg[t] = the smallest el of row t); the kernel brings every
//             block to 2^eg[t] and its epilogue multiplies by 2^-eg[t]
//   eg_out, el_out  the same exponents for planes this kernel writes
//             (gate/up: h); eg_out and the el_out rows must be 0 before
//             the kernel (only nonzero block exponents are written)
//   range_flag set to 1 when a value split here is outside the pair's range
//             (|v| >= 2^15 or not finite): its products are then not exact
struct ActScale {
    const float *rs = nullptr;
    const int *eg = nullptr;
    const int8_t *el = nullptr;
    int el_stride = 0;          // blocks per row of el / el_out
    int *eg_out = nullptr;
    int8_t *el_out = nullptr;
    uint32_t *range_flag = nullptr;
};

// MFMA matrix-matrix path (prefill with T >= kGemmMinTokens tokens). Activations
// are passed as an f16 hi plane [T][K] followed by an f16 lo plane (a_split),
// or as f32 [T][K].
// rs (if set) receives each row's factor 2^-e of the scaled planes (see
// ActScale); eg_zero (if set) is cleared for each row, and el_zero's el_n
// bytes of each row with it.
hipError_t launch_rms_split(float *x, int T, int K, const float *w, float eps, _Float16 *u,
                            const float *part, int splits, hipStream_t s, float *rs = nullptr,
                            int *eg_zero = nullptr, int8_t *el_zero = nullptr, int el_n = 0);
// Split-K for short prompts: when the plain GEMM would launch only a few
// workgroups (each walking all of K), the K steps are split over
// gemm_splitk(N, K, T) > 1 slices that write partial sums part[z][T][N];
// launch_rms_split (or its add-only form, u = NULL) then adds them to x.
constexpr int kSplitKMax = 8;
constexpr int kSplitKMaxTokens = 1024;
int gemm_splitk(int N, int K, int T);
// Longest prompt for which an N-row product may be split: the partial-sum
// scratch holds kSplitKMax * gemm_splitk_max_tokens(N) * N floats.
int gemm_splitk_max_tokens(int N);
// W in Q8_0 or Q5_0 (fmt).
hipError_t launch_gemm_part(const uint8_t *W, int N, int K, const _Float16 *A, int T, int splits, float *part,
                            hipStream_t s, const ActScale &sc = ActScale{}, int fmt = F_Q8_0);
hipError_t launch_gemm_matmul(const uint8_t *W, int N, int K, const void *A, bool a_split, int T,
                              int accumulate, float *Y, hipStream_t s, const ActScale &sc = ActScale{},
                              int fmt = F_Q8_0);
hipError_t launch_gemm_qkv(const Dims &d, const LayerPtrs &w, const _Float16 *u, const StepState *st,
                           const float2 *rope, float *q, float *kc, float *vc, int T, hipStream_t s,
                           const ActScale &sc = ActScale{});
hipError_t launch_gemm_gateup(const Dims &d, const LayerPtrs &w, const _Float16 *u, _Float16 *h, int T,
                              hipStream_t s, const ActScale &sc = ActScale{});

// Q4_K / Q6_K matrices (N rows of K weights, K % 256 == 0). One token: the
// VALU GEMV; several: the MFMA GEMM (activations f32, or split planes).
// Y[t] (+)= W X[t].
hipError_t launch_kq_gemv(int fmt, const uint8_t *W, int N, int K, const float *X, int accumulate, float *Y,
                          hipStream_t s);
hipError_t launch_gemm_kq(int fmt, const uint8_t *W, int N, int K, const void *A, bool a_split, int T,
                          int accumulate, float *Y, hipStream_t s, const ActScale &sc = ActScale{});

// Prefill attention: T queries, causal mask offset by the cached prefix.
struct AttnPrefillArgs {
    const float *q;        // [T][nh][hd]
    const float *kc, *vc;  // [nkv][kv_stride][hd]
    float *o;              // [T][nh][hd] f32, or (o_split set) unused
    _Float16 *o_split;     // when set: f16 hi plane [T][nh*hd], then the lo plane
    int T, kv_len, kv_stride, nh, nkv, hd;
    float scale;
    uint32_t *range_flag = nullptr;  // set to 1 when a value split into an f16 pair is out of its range
    // Key-split partials (NULL: every query block's keys in one workgroup).
    // With it, query blocks with more than pf_chunk key blocks of 64 are cut
    // into key ranges of pf_chunk blocks, each a workgroup writing (max,
    // sum, unnormalised o) per query to pf_part [nh][T][kMaxPfSplits][hd + 2];
    // a merge kernel then writes o.
    float *pf_part = nullptr;
    int pf_chunk = 0;
};
constexpr int kMaxPfSplits = 4;   // key ranges per query block at most
// Key blocks per range for a prefill of kv_len keys (0: no split).
int attn_prefill_chunk(int kv_len);
hipError_t launch_attn_prefill(const AttnPrefillArgs &a, hipStream_t s);

}  // namespace q8l
